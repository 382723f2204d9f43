// Embedding forward and backward ([LS2] sec. 2.1.2).
//
// Forward:  out[t] = Dropout(s * E[id_t] + P[t mod L]) -- a row gather fused
// with the scale, the position add and the dropout, one pass over the output.
//
// Backward: dE[w] += s * sum_{t: id_t = w} m_t * dy_t with the dropout mask
// m regenerated from (seed, offset).  Repeated ids collide on one row of dE,
// and, as in [LS2] sec. 2.1.2, the collisions are summed with fp32 atomic
// adds -- after each wave has added up the repeats inside its own chunk of
// tokens, and with every atomic instruction covering 64 consecutive floats.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int LPR, int NCH, bool DROP>
__global__ __launch_bounds__(kBlock) void emb_fwd_vec_kernel(half_t* out, const int32_t* ids,
                                                             const half_t* E, const half_t* P,
                                                             uint32_t tokens, uint32_t h,
                                                             uint32_t vocab, FastDiv seq,
                                                             float scale, Dropout d) {
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l = lane % LPR;
    const int sub = lane / LPR;
    const uint32_t nv = h / 8;
    for (uint32_t t0 = blockIdx.x * (kWaves * RPW); t0 < tokens; t0 += gridDim.x * (kWaves * RPW)) {
        const uint32_t t = t0 + wave * RPW + sub;
        if (t >= tokens) continue;
        const int32_t id = ids[t];
        const bool valid = id >= 0 && static_cast<uint32_t>(id) < vocab;
        const uint32_t pos = seq.mod(t);
        const half8* erow = reinterpret_cast<const half8*>(E + static_cast<size_t>(valid ? id : 0) * h);
        const half8* prow = reinterpret_cast<const half8*>(P + static_cast<size_t>(pos) * h);
        half8* orow = reinterpret_cast<half8*>(out + static_cast<size_t>(t) * h);
        half8 ev[NCH], pv[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t cv = l + j * LPR;
            if (cv < nv) {
                if (valid) ev[j] = erow[cv];
                pv[j] = prow[cv];
            }
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t cv = l + j * LPR;
            if (cv < nv) {
                float o[8];
                if (valid) {
                    float e[8], p[8], f[8];
                    unpack8(ev[j], e);
                    unpack8(pv[j], p);
                    if (DROP) {
                        dropout_factors8(d, static_cast<uint64_t>(t) * nv + cv, f);
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; ++k) f[k] = 1.0f;
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) o[k] = fmaf(scale, e[k], p[k]) * f[k];
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) o[k] = __builtin_nanf("");
                }
                __builtin_nontemporal_store(pack8(o), orow + cv);   // written once: stream it
            }
        }
    }
}

// Element-wise fallback (unaligned tables or hidden % 8 != 0).
template <bool DROP>
__global__ __launch_bounds__(kBlock) void emb_fwd_scalar_kernel(half_t* out, const int32_t* ids,
                                                                const half_t* E, const half_t* P,
                                                                uint64_t n, uint32_t h,
                                                                uint32_t vocab, uint32_t seq,
                                                                float scale, Dropout d) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const uint64_t t = i / h;
        const uint32_t c = static_cast<uint32_t>(i - t * h);
        const int32_t id = ids[t];
        float o;
        if (id >= 0 && static_cast<uint32_t>(id) < vocab) {
            const float e = static_cast<float>(E[static_cast<size_t>(id) * h + c]);
            const float p = static_cast<float>(P[static_cast<size_t>(t % seq) * h + c]);
            o = fmaf(scale, e, p) * (DROP ? dropout_factor1(d, i) : 1.0f);
        } else {
            o = __builtin_nanf("");
        }
        out[i] = static_cast<half_t>(o);
    }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
// A wave takes a chunk of 64 consecutive tokens and one slice of 512 columns
// (lane l owns the 8 consecutive columns 8l..8l+7 of the slice, so its dy
// loads are 16 bytes and one Philox call gives its 8 dropout decisions).
// The chunk's ids are sorted inside the wave (bitonic network over lane
// shuffles), so the tokens of one id arrive back to back and are summed in
// registers.  At the end of each run of equal ids the wave writes its sum
// to LDS and reads it back transposed -- lane l then holds columns l, l+64,
// ..., l+448 -- so every fp32 atomic add instruction covers 64 consecutive
// floats of the dE row.  Atomics are the only cross-wave combination
// ([LS2] sec. 2.1.2); their order is not fixed.
constexpr int kChunk = 64;                // tokens per wave (one key per lane)
constexpr int kSliceCols = kWave * 8;     // columns per wave
constexpr int kBatch = 16;                // dy rows in flight per lane
constexpr uint64_t kNoToken = ~0ull;

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <bool DROP>
__global__ __launch_bounds__(kBlock) void emb_bwd_kernel(float* dE, const int32_t* ids,
                                                         const half_t* dy, uint32_t tokens,
                                                         uint32_t h, uint32_t vocab, uint32_t slices,
                                                         float scale, Dropout d) {
    __shared__ float xpose[kWaves][kSliceCols];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t item = blockIdx.x * kWaves + wave;
    const uint32_t chunk = item / slices, sl = item - chunk * slices;
    const uint32_t t0 = chunk * kChunk;
    if (t0 >= tokens) return;
    const uint32_t nv = h / 8;
    const uint32_t cv = sl * kWave + lane;            // this lane's 8-column vector
    const bool active = cv < nv;
    float* xp = xpose[wave];

    // Keys (id << 8 | local token); invalid ids and the ragged tail sort last.
    uint64_t key = kNoToken;
    if (t0 + lane < tokens) {
        const int32_t id = ids[t0 + lane];
        if (id >= 0 && static_cast<uint32_t>(id) < vocab)
            key = (static_cast<uint64_t>(id) << 8) | static_cast<uint32_t>(lane);
    }
    key = wave_sort_asc(key, lane);
    const uint64_t next = __shfl_down(static_cast<unsigned long long>(key), 1);
    const uint64_t ends = __ballot(lane == kWave - 1 || (next >> 8) != (key >> 8));
    const int count = __popcll(__ballot(key != kNoToken));

    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    for (int b0 = 0; b0 < count; b0 += kBatch) {
        half8 g[kBatch];
        uint32_t tk[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            tk[j] = 0;
            if (b0 + j < count) {
                tk[j] = t0 + static_cast<uint32_t>(readlane_u64(key, b0 + j) & 0xFF);
                if (active) g[j] = reinterpret_cast<const half8*>(dy + static_cast<size_t>(tk[j]) * h)[cv];
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int pos = b0 + j;
            if (pos >= count) break;
            if (active) {
                float gf[8], f[8];
                unpack8(g[j], gf);
                if (DROP) {
                    dropout_factors8(d, static_cast<uint64_t>(tk[j]) * nv + cv, f);
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) f[k] = 1.0f;
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = fmaf(gf[k] * f[k], scale, acc[k]);
            }
            if ((ends >> pos) & 1ull) {
                // Transpose through LDS, then coalesced atomics on the id's row.
                const uint32_t id = static_cast<uint32_t>(readlane_u64(key, pos) >> 8);
                float4v* w = reinterpret_cast<float4v*>(xp + lane * 8);
                w[0] = float4v{acc[0], acc[1], acc[2], acc[3]};
                w[1] = float4v{acc[4], acc[5], acc[6], acc[7]};
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                float* row = dE + static_cast<size_t>(id) * h + static_cast<size_t>(sl) * kSliceCols;
                const uint32_t cols = h - sl * kSliceCols;        // columns of this slice present
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t c = k * kWave + lane;
                    if (c < cols) unsafeAtomicAdd(row + c, xp[c]);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
            }
        }
    }
}

// Element-wise fallback (unaligned or hidden % 8 != 0): one fp32 atomic per
// element, consecutive lanes on consecutive columns.
template <bool DROP>
__global__ __launch_bounds__(kBlock) void emb_bwd_scalar_kernel(float* dE, const int32_t* ids,
                                                                const half_t* dy, uint64_t n,
                                                                uint32_t h, uint32_t vocab,
                                                                float scale, Dropout d) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const uint64_t t = i / h;
        const uint32_t c = static_cast<uint32_t>(i - t * h);
        const int32_t id = ids[t];
        if (id < 0 || static_cast<uint32_t>(id) >= vocab) continue;
        const float f = DROP ? dropout_factor1(d, i) : 1.0f;
        unsafeAtomicAdd(dE + static_cast<size_t>(id) * h + c, static_cast<float>(dy[i]) * f * scale);
    }
}

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* p, uint64_t n) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    const uint64_t n4 = (reinterpret_cast<uintptr_t>(p) & 15u) == 0 ? n / 4 : 0;
    float4v* p4 = reinterpret_cast<float4v*>(p);
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    for (uint64_t i = tid; i < n4; i += stride) p4[i] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (uint64_t i = n4 * 4 + tid; i < n; i += stride) p[i] = 0.0f;
}

unsigned grid_cap(uint64_t blocks, unsigned cap) {
    return static_cast<unsigned>(blocks == 0 ? 1 : (blocks < cap ? blocks : cap));
}

struct EmbShape {
    int lpr, nch;
    const char* name;
};

bool emb_shape(int64_t h, EmbShape* s) {
    const int64_t nv = h / 8;
    if (nv <= 8) *s = {8, 1, "lpr8_nch1"};
    else if (nv <= 16) *s = {16, 1, "lpr16_nch1"};
    else if (nv <= 32) *s = {16, 2, "lpr16_nch2"};
    else if (nv <= 64) *s = {32, 2, "lpr32_nch2"};
    else if (nv <= 96) *s = {32, 3, "lpr32_nch3"};
    else if (nv <= 128) *s = {64, 2, "lpr64_nch2"};
    else if (nv <= 256) *s = {64, 4, "lpr64_nch4"};
    else if (nv <= 512) *s = {64, 8, "lpr64_nch8"};
    else return false;
    return true;
}

#define LS_EMB_FWD(LPR, NCH)                                                                    \
    do {                                                                                        \
        if (drop)                                                                               \
            emb_fwd_vec_kernel<LPR, NCH, true><<<grid, kBlock, 0, st>>>(o16, ids, E16, P16, t32, h32, v32, sdiv, scale, d); \
        else                                                                                    \
            emb_fwd_vec_kernel<LPR, NCH, false><<<grid, kBlock, 0, st>>>(o16, ids, E16, P16, t32, h32, v32, sdiv, scale, d); \
    } while (0)

}  // namespace
}  // namespace ls

extern "C" {

int ls_embedding_fwd(void* out, const int32_t* ids, const void* tok_emb, const void* pos_emb,
                     int64_t batch, int64_t seq_len, int64_t hidden, int64_t vocab,
                     int64_t max_pos, float scale, float p, uint64_t seed, uint64_t offset,
                     void* stream) {
    using namespace ls;
    const char* name = "ls_embedding_fwd";
    if (batch < 0 || seq_len < 0 || hidden < 0 || vocab < 0 || max_pos < 0)
        return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    Dropout d;
    if (!make_dropout(p, seed, offset, &d))
        return fail(LS_ERR_PARAM, "%s: dropout probability %g outside [0, 1]", name, (double)p);
    if (!host_finite(scale)) return fail(LS_ERR_PARAM, "%s: scale must be finite", name);
    if (batch == 0 || seq_len == 0 || hidden == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (max_pos < seq_len) return fail(LS_ERR_SHAPE, "%s: max_pos %lld < seq_len %lld", name,
                                       (long long)max_pos, (long long)seq_len);
    if (vocab >= (1ll << 31) || hidden >= (1ll << 31) || batch > INT32_MAX / seq_len)
        return fail(LS_ERR_SHAPE, "%s: sizes must be < 2^31", name);
    if (!out || !ids || !pos_emb || (vocab > 0 && !tok_emb)) return fail(LS_ERR_NULL, "%s: null pointer", name);
    const int64_t tokens = batch * seq_len;
    const bool drop = d.thr != 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* o16 = static_cast<half_t*>(out);
    auto* E16 = static_cast<const half_t*>(tok_emb);
    auto* P16 = static_cast<const half_t*>(pos_emb);
    const uint32_t t32 = static_cast<uint32_t>(tokens), h32 = static_cast<uint32_t>(hidden),
                   v32 = static_cast<uint32_t>(vocab);
    EmbShape s;
    const bool vec = hidden % 8 == 0 && aligned16(out) && aligned16(tok_emb) && aligned16(pos_emb) &&
                     emb_shape(hidden, &s);
    clear_hip_error();
    if (vec) {
        const FastDiv sdiv(static_cast<uint32_t>(seq_len));
        const int64_t per_block = kWaves * (kWave / s.lpr);
        const unsigned grid = grid_cap((tokens + per_block - 1) / per_block, 1u << 20);
        if (s.lpr == 8) LS_EMB_FWD(8, 1);
        else if (s.lpr == 16 && s.nch == 1) LS_EMB_FWD(16, 1);
        else if (s.lpr == 16) LS_EMB_FWD(16, 2);
        else if (s.lpr == 32 && s.nch == 2) LS_EMB_FWD(32, 2);
        else if (s.lpr == 32) LS_EMB_FWD(32, 3);
        else if (s.nch == 2) LS_EMB_FWD(64, 2);
        else if (s.nch == 4) LS_EMB_FWD(64, 4);
        else LS_EMB_FWD(64, 8);
        char buf[96];
        snprintf(buf, sizeof(buf), "embedding_fwd/%s%s", s.name, drop ? "" : "_p0");
        set_dispatch(buf);
    } else {
        const uint64_t n = static_cast<uint64_t>(tokens) * static_cast<uint64_t>(hidden);
        const unsigned grid = grid_cap((n + kBlock - 1) / kBlock, 65536);
        if (drop)
            emb_fwd_scalar_kernel<true><<<grid, kBlock, 0, st>>>(o16, ids, E16, P16, n, h32, v32,
                                                                 static_cast<uint32_t>(seq_len), scale, d);
        else
            emb_fwd_scalar_kernel<false><<<grid, kBlock, 0, st>>>(o16, ids, E16, P16, n, h32, v32,
                                                                  static_cast<uint32_t>(seq_len), scale, d);
        set_dispatch("embedding_fwd/scalar");
    }
    return launch_status(name);
}

int ls_embedding_bwd(float* grad_tok_emb, const int32_t* ids, const void* dy, int64_t batch,
                     int64_t seq_len, int64_t hidden, int64_t vocab, float scale, float p,
                     uint64_t seed, uint64_t offset, int zero_first, void* stream) {
    using namespace ls;
    const char* name = "ls_embedding_bwd";
    if (batch < 0 || seq_len < 0 || hidden < 0 || vocab < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    Dropout d;
    if (!make_dropout(p, seed, offset, &d))
        return fail(LS_ERR_PARAM, "%s: dropout probability %g outside [0, 1]", name, (double)p);
    if (!host_finite(scale)) return fail(LS_ERR_PARAM, "%s: scale must be finite", name);
    if (vocab >= (1ll << 31) || hidden >= (1ll << 31) || (seq_len > 0 && batch > INT32_MAX / seq_len))
        return fail(LS_ERR_SHAPE, "%s: sizes must be < 2^31", name);
    const int64_t tokens = batch * seq_len;
    const uint64_t table = static_cast<uint64_t>(vocab) * static_cast<uint64_t>(hidden);
    if (table == 0 || (tokens == 0 && !zero_first)) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!grad_tok_emb || (tokens > 0 && (!ids || !dy))) return fail(LS_ERR_NULL, "%s: null pointer", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    clear_hip_error();
    if (zero_first) {
        fill_zero_kernel<<<grid_cap((table / 4 + kBlock - 1) / kBlock, 8192), kBlock, 0, st>>>(grad_tok_emb, table);
        const int rc = launch_status(name);
        if (rc != LS_OK || tokens == 0) {
            set_dispatch("embedding_bwd/zero_only");
            return rc;
        }
    }
    const bool drop = d.thr != 0;
    const uint32_t t32 = static_cast<uint32_t>(tokens), h32 = static_cast<uint32_t>(hidden),
                   v32 = static_cast<uint32_t>(vocab);
    auto* dy16 = static_cast<const half_t*>(dy);
    if (hidden % 8 == 0 && aligned16(dy)) {
        const uint32_t slices = (h32 + kSliceCols - 1) / kSliceCols;
        const uint64_t items = static_cast<uint64_t>((t32 + kChunk - 1) / kChunk) * slices;
        const unsigned grid = static_cast<unsigned>((items + kWaves - 1) / kWaves);
        if (drop) emb_bwd_kernel<true><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
        else emb_bwd_kernel<false><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
        set_dispatch("embedding_bwd/chunk64_sorted_atomic");
    } else {
        const uint64_t n = static_cast<uint64_t>(tokens) * static_cast<uint64_t>(hidden);
        const unsigned grid = grid_cap((n + kBlock - 1) / kBlock, 65536);
        if (drop) emb_bwd_scalar_kernel<true><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, n, h32, v32, scale, d);
        else emb_bwd_scalar_kernel<false><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, n, h32, v32, scale, d);
        set_dispatch("embedding_bwd/atomic_elementwise");
    }
    return launch_status(name);
}

}  // extern "C"
