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
        out[i] = to_half(o);
    }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
// dE rows are combined with fp32 atomic adds ([LS2] sec. 2.1.2), so the
// kernels first add up, in registers, the gradients of tokens that share an
// id -- over as many tokens as is cheap: atomics cost about one float per
// channel clock, and a Zipf-like id law puts a large share of the tokens on a
// few rows, whose atomics also serialise on their addresses.
//
// In both kernels below a wave works on one slice of 512 columns (lane l owns
// the 8 consecutive columns 8l..8l+7 of the slice, so its dy loads are 16
// bytes and one Philox call gives its 8 dropout decisions) and visits tokens
// in id order, so the tokens of one id arrive back to back.  At the end of
// each run of equal ids the wave writes its sum to LDS and reads it back
// transposed -- lane l then holds columns l, l+64, ..., l+448 -- so every
// atomic add instruction covers 64 consecutive floats of the dE row.  Atomics
// are the only combination across waves; their order is not fixed.
//
// Wide vocabularies (ids of 22 bits or more): a wave sorts the ids of 64
// consecutive tokens itself (bitonic network over lane shuffles, 64-bit keys)
// and walks all of them.
constexpr int kChunk = 64;                // tokens per wave (one key per lane)
constexpr int kSliceCols = kWave * 8;     // columns per wave
constexpr int kBatch = 16;                // dy rows in flight per lane
constexpr uint64_t kNoToken = ~0ull;

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), lane);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Adds a run's sum (acc: this lane's 8 columns) to row id of dE, slice sl:
// transposed through the wave's 512-float LDS buffer xp, then 8 atomic add
// instructions of 64 consecutive floats.  Leaves acc zeroed.
__device__ __forceinline__ void flush_row(float* dE, uint32_t id, uint32_t h, uint32_t sl, float* xp,
                                          float (&acc)[8], int lane) {
    float4v* w = reinterpret_cast<float4v*>(xp + lane * 8);
    w[0] = float4v{acc[0], acc[1], acc[2], acc[3]};
    w[1] = float4v{acc[4], acc[5], acc[6], acc[7]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float v[8];                                       // all 8 reads, then one wait
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xp[k * kWave + lane];
    float* row = dE + static_cast<size_t>(id) * h + static_cast<size_t>(sl) * kSliceCols;
    const uint32_t cols = h - sl * kSliceCols;        // columns of this slice present
    if (cols >= static_cast<uint32_t>(kSliceCols)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) unsafeAtomicAdd(row + k * kWave + lane, v[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t c = k * kWave + lane;
            if (c < cols) unsafeAtomicAdd(row + c, v[k]);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
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
        for (int j = 0; j < kBatch; ++j) g[j] = half8{};      // filled first: the loads stay in flight
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
                const uint32_t id = static_cast<uint32_t>(readlane_u64(key, pos) >> 8);
                flush_row(dE, id, h, sl, xp, acc, lane);
            }
        }
    }
}

// Ids below 2^22: a block of kSortThreads threads takes a chunk of kSortChunk
// consecutive tokens and one column slice, and sorts the chunk's
// (id << 10 | position) keys in LDS.  Each of its waves then walks
// kWavePos consecutive sorted positions, so runs are summed over up to 1024
// tokens instead of 64 (on Zipf(1.1) ids at 8192 tokens: 3.9M atomic floats
// instead of 6.0M, and at most 76 flushes instead of 128 on the most frequent
// row), while 16 positions per wave keep every wave's chain of dependent
// loads short.  Every block that works on a chunk (one per slice and group
// of 64 positions) sorts it again: a few thousand cycles of ALU at the start
// of each block, which keeps the call one launch without a workspace.
constexpr int kSortThreads = 256;
constexpr int kSortChunk = 1024;
constexpr int kSortPer = kSortChunk / kSortThreads;      // keys per thread
constexpr int kWavePos = 16;                             // sorted positions per wave
constexpr int kBlockPos = kWavePos * (kSortThreads / kWave);
constexpr int kParts = kSortChunk / kBlockPos;            // blocks per chunk and slice
constexpr int kPosBits = 10;                              // log2(kSortChunk)
constexpr uint32_t kNoKey = 0xFFFFFFFFu;                  // invalid id or past the end
constexpr int64_t kSortMaxVocab = (1ll << (32 - kPosBits)) - 1;   // ids < 2^22 - 1: keys below kNoKey
static_assert(kSortChunk == 1 << kPosBits, "position field");

// Bitonic sort, ascending, of the block's kSortChunk keys; thread t holds
// positions kSortPer*t .. kSortPer*t + kSortPer-1 in k.  Compare-exchange
// partners at distance j sit in the same thread (j < kSortPer), in another
// lane of the same wave (j < kSortPer*64: one DPP / swizzle / permute per key) or in another
// wave (through lds, between two barriers).
__device__ __forceinline__ uint32_t bitonic_pick(uint32_t i, uint32_t j, uint32_t size, uint32_t a,
                                                 uint32_t b) {
    const bool lower = (i & j) == 0, asc = (i & size) == 0;
    return lower == asc ? min(a, b) : max(a, b);
}

__device__ __forceinline__ void block_sort_asc(uint32_t (&k)[kSortPer], uint32_t* lds) {
    const uint32_t base = threadIdx.x * kSortPer;
    constexpr uint32_t kWaveSpan = kSortPer * kWave;
#pragma unroll
    for (uint32_t size = 2; size <= kSortChunk; size <<= 1) {
#pragma unroll
        for (uint32_t j = size >> 1; j > 0; j >>= 1) {
            if (j >= kWaveSpan) {
                __syncthreads();
#pragma unroll
                for (int r = 0; r < kSortPer; ++r) lds[base + r] = k[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < kSortPer; ++r) k[r] = bitonic_pick(base + r, j, size, k[r], lds[(base + r) ^ j]);
            } else if (j >= kSortPer) {
#pragma unroll
                for (int r = 0; r < kSortPer; ++r) {
                    const uint32_t o = lane_xor_u32(k[r], j / kSortPer);
                    k[r] = bitonic_pick(base + r, j, size, k[r], o);
                }
            } else {
#pragma unroll
                for (int r = 0; r < kSortPer; ++r) {
                    if (r & j) continue;
                    const uint32_t a = k[r], b = k[r | j];
                    const bool asc = ((base + r) & size) == 0;
                    k[r] = asc ? min(a, b) : max(a, b);
                    k[r | j] = asc ? max(a, b) : min(a, b);
                }
            }
        }
    }
}

template <bool DROP>
__global__ __launch_bounds__(kSortThreads) void emb_bwd_sorted_kernel(float* dE, const int32_t* ids,
                                                                    const half_t* dy, uint32_t tokens,
                                                                    uint32_t h, uint32_t vocab,
                                                                    uint32_t slices, float scale,
                                                                    Dropout d) {
    __shared__ uint32_t keys[kSortChunk];
    __shared__ float xpose[kSortThreads / kWave][kSliceCols];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t sl = blockIdx.x % slices, rest = blockIdx.x / slices;
    const uint32_t part = rest % kParts, chunk = rest / kParts;
    const uint32_t c0 = chunk * kSortChunk;
    const uint32_t n = min(static_cast<uint32_t>(kSortChunk), tokens - c0);
    if (part * kBlockPos >= n) return;                 // the whole block: no position of its group exists

    // All id loads before the first wait: unconditional, at positions
    // clamped to the chunk (n >= 1 here); past the end is marked afterwards.
    int32_t raw[kSortPer];
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) raw[r] = ids[c0 + min(threadIdx.x * kSortPer + r, n - 1)];
    uint32_t k[kSortPer];
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) {
        const uint32_t pos = threadIdx.x * kSortPer + r;
        const bool ok = pos < n && raw[r] >= 0 && static_cast<uint32_t>(raw[r]) < vocab;
        k[r] = ok ? (static_cast<uint32_t>(raw[r]) << kPosBits) | pos : kNoKey;
    }
    block_sort_asc(k, keys);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortPer; ++r) keys[threadIdx.x * kSortPer + r] = k[r];
    __syncthreads();

    const uint32_t q0 = part * kBlockPos + static_cast<uint32_t>(wave) * kWavePos;
    const uint32_t nv = h / 8;
    const uint32_t cv = sl * kWave + lane;            // this lane's 8-column vector
    const bool active = cv < nv;
    float* xp = xpose[wave];
    uint32_t key[kWavePos + 1];
#pragma unroll
    for (int j = 0; j <= kWavePos; ++j)
        key[j] = __builtin_amdgcn_readfirstlane(q0 + j < kSortChunk ? keys[q0 + j] : kNoKey);
    if (key[0] == kNoKey) return;                    // invalid keys sort last: nothing left for this wave

    // Every load of the wave's tokens before the first wait: zero-filled
    // registers, then the loads of the valid positions.
    half8 g[kWavePos];
#pragma unroll
    for (int j = 0; j < kWavePos; ++j) g[j] = half8{};
#pragma unroll
    for (int j = 0; j < kWavePos; ++j) {
        if (key[j] != kNoKey && active) {
            const uint32_t t = c0 + (key[j] & (kSortChunk - 1));
            g[j] = reinterpret_cast<const half8*>(dy + static_cast<size_t>(t) * h)[cv];
        }
    }
    // The Philox words depend on the token only: computed while the loads
    // are in flight.
    uint32_t pw[kWavePos][4];
    if (DROP) {
#pragma unroll
        for (int j = 0; j < kWavePos; ++j) {
            const uint32_t t = c0 + (key[j] & (kSortChunk - 1));
            if (key[j] != kNoKey) dropout_words(d, static_cast<uint64_t>(t) * nv + cv, pw[j]);
        }
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kWavePos; ++j) {
        if (key[j] == kNoKey) break;
        float gf[8], f[8];
        unpack8(g[j], gf);
        if (DROP) {
            dropout_factors_from(d, pw[j], f);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = 1.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(gf[e] * f[e], scale, acc[e]);
        // A run ends at the wave's last position or where the id changes
        // (kNoKey has an id field above every valid id).
        if (j == kWavePos - 1 || (key[j + 1] >> kPosBits) != (key[j] >> kPosBits))
            flush_row(dE, key[j] >> kPosBits, h, sl, xp, acc, lane);
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
        if (vocab <= kSortMaxVocab) {
            const uint64_t blocks = static_cast<uint64_t>((t32 + kSortChunk - 1) / kSortChunk) * kParts * slices;
            if (blocks > 0x7FFFFFFFull) return fail(LS_ERR_SHAPE, "%s: tokens x hidden too large", name);
            const unsigned grid = static_cast<unsigned>(blocks);
            if (drop)
                emb_bwd_sorted_kernel<true><<<grid, kSortThreads, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
            else
                emb_bwd_sorted_kernel<false><<<grid, kSortThreads, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
            set_dispatch("embedding_bwd/sorted1024_atomic");
        } else {
            const uint64_t items = static_cast<uint64_t>((t32 + kChunk - 1) / kChunk) * slices;
            if ((items + kWaves - 1) / kWaves > 0x7FFFFFFFull) return fail(LS_ERR_SHAPE, "%s: tokens x hidden too large", name);
            const unsigned grid = static_cast<unsigned>((items + kWaves - 1) / kWaves);
            if (drop) emb_bwd_kernel<true><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
            else emb_bwd_kernel<false><<<grid, kBlock, 0, st>>>(grad_tok_emb, ids, dy16, t32, h32, v32, slices, scale, d);
            set_dispatch("embedding_bwd/chunk64_sorted_atomic");
        }
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
