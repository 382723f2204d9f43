// Row softmax forward and backward over attention scores ([L10] slides 23-26).
//
// The slides tune the launch shape to the row length instead of changing the
// formula: short rows share a thread group, long rows get more elements per
// thread, and the parameters are compile-time template arguments picked at
// call time.  Here the same idea is laid out for 64-lane wavefronts: a row
// belongs to an aligned group of LPR lanes (LPR = 8..64, so one wave holds
// 64/LPR rows) and each lane keeps NCH chunks of CW elements in registers
// (CW = 8 is one 16-byte access).  The two dependent row reductions of the
// forward (max, then sum of exponentials) and the one of the backward
// (sum y*dy) are DPP/swizzle butterflies inside the lane group, with no LDS
// and no block barrier.  Rows too long for one wave's registers use a
// 1024-thread block per row, combining the waves' partial results through
// LDS.
//
// Masking: keys j >= key_lengths[b] and, for causal rows, keys j > i are
// excluded from max and sum and written as exact zeros; chunks lying wholly
// in the masked tail are not read at all.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;

template <int CW>
struct Chunk;
// Score rows are streamed once: non-temporal 16-byte loads and stores.
// Loads go into raw registers filled beforehand (fill(), then a conditional
// load()), so nothing writes them after the load and all loads of a row are
// in flight before the first wait; widen() converts once they are needed.
template <>
struct Chunk<8> {
    using T = half8;
    static __device__ __forceinline__ T fill(float v) {
        const half_t h = static_cast<half_t>(v);
        return half8{h, h, h, h, h, h, h, h};
    }
    static __device__ __forceinline__ T load(const half_t* p, size_t i) {
        return __builtin_nontemporal_load(reinterpret_cast<const half8*>(p + i));
    }
    static __device__ __forceinline__ void widen(const T& r, float f[8]) { unpack8(r, f); }
    static __device__ __forceinline__ void store(half_t* p, size_t i, const float f[8]) {
        __builtin_nontemporal_store(pack8(f), reinterpret_cast<half8*>(p + i));
    }
};
// Element-wise path: one fp16 element per 32-bit register (zero-extended);
// two to a register would need each load merged into its pair as it arrives.
template <>
struct Chunk<1> {
    using T = uint32_t;
    static __device__ __forceinline__ T fill(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<half_t>(v));
    }
    static __device__ __forceinline__ T load(const half_t* p, size_t i) {
        return reinterpret_cast<const uint16_t*>(p)[i];
    }
    static __device__ __forceinline__ void widen(const T& r, float f[1]) {
        f[0] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(r)));
    }
    static __device__ __forceinline__ void store(half_t* p, size_t i, const float f[1]) {
        p[i] = to_half(f[0]);
    }
};

struct RowMask {
    const int32_t* key_len;   // [batch] or null
    int causal;
    FastDiv q_len;            // row -> query index i = row % q_len
    FastDiv per_batch;        // row -> batch b = row / (heads * q_len)
};

// Number of leading valid keys of a row (the valid set is always a prefix).
template <bool MASKED>
__device__ __forceinline__ uint32_t valid_keys(const RowMask& m, uint32_t row, uint32_t k) {
    if (!MASKED) return k;
    uint32_t n = k;
    if (m.key_len) {
        const int32_t len = m.key_len[m.per_batch.div(row)];
        n = len <= 0 ? 0u : (static_cast<uint32_t>(len) < k ? static_cast<uint32_t>(len) : k);
    }
    if (m.causal) {
        const uint32_t lim = m.q_len.mod(row) + 1;
        n = lim < n ? lim : n;
    }
    return n;
}

// ---------------------------------------------------------------------------
// One row per LPR-lane group
// ---------------------------------------------------------------------------
template <int LPR, int NCH, int CW, bool MASKED>
__global__ __launch_bounds__(kBlock) void softmax_fwd_kernel(half_t* y, const half_t* x,
                                                             uint32_t rows, uint32_t k,
                                                             RowMask mask) {
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l = lane % LPR;
    const int sub = lane / LPR;
    for (uint32_t r0 = blockIdx.x * (kWaves * RPW); r0 < rows; r0 += gridDim.x * (kWaves * RPW)) {
        const uint32_t row = r0 + wave * RPW + sub;
        const bool ok = row < rows;
        const size_t base = static_cast<size_t>(row) * k;
        typename Chunk<CW>::T raw[NCH];
        uint32_t n;
        if constexpr (CW == 1) {
            // Element-wise path: unconditional loads at indices clamped into
            // the tensor (issued before the key length is read), then -inf
            // past the valid keys (a load under a branch gets its conversion
            // moved into the branch: a wait per element).
            const size_t cbase = static_cast<size_t>(ok ? row : rows - 1) * k;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = l + j * LPR;
                raw[j] = Chunk<CW>::load(x, cbase + (c < k ? c : k - 1));
            }
            n = ok ? valid_keys<MASKED>(mask, row, k) : 0u;
#pragma unroll
            for (int j = 0; j < NCH; ++j) raw[j] = l + j * LPR < n ? raw[j] : Chunk<CW>::fill(-INFINITY);
        } else if constexpr (!MASKED) {
            // Every key valid: unconditional loads, chunks past the row end
            // redirected to its last vector (a cache hit) and set to -inf.
            n = ok ? k : 0u;
            const size_t cbase = static_cast<size_t>(ok ? row : rows - 1) * k;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                raw[j] = Chunk<CW>::load(x, cbase + (c < k ? c : k - CW));
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) raw[j] = (l + j * LPR) * CW < n ? raw[j] : Chunk<CW>::fill(-INFINITY);
        } else {
            // Masked rows: keys past the row's length are not read at all.
            n = ok ? valid_keys<MASKED>(mask, row, k) : 0u;
#pragma unroll
            for (int j = 0; j < NCH; ++j) raw[j] = Chunk<CW>::fill(-INFINITY);
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                if (c < n) raw[j] = Chunk<CW>::load(x, base + c);
            }
        }
        float v[NCH][CW];
#pragma unroll
        for (int j = 0; j < NCH; ++j) Chunk<CW>::widen(raw[j], v[j]);
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int q = 0; q < CW; ++q) {
                if (MASKED && (l + j * LPR) * CW + q >= n) v[j][q] = -INFINITY;
                m = fmaxf(m, v[j][q]);
            }
        m = group_max<LPR>(m);
        if (!(m > -INFINITY)) m = 0.0f;    // no valid key, or all valid keys are -inf: row of zeros
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int q = 0; q < CW; ++q) {
                v[j][q] = __builtin_amdgcn_exp2f((v[j][q] - m) * kLog2e);
                s += v[j][q];
            }
        s = group_sum<LPR>(s);
        const float inv = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (l + j * LPR) * CW;
            if (ok && c < k) {
                float o[CW];
#pragma unroll
                for (int q = 0; q < CW; ++q) o[q] = v[j][q] * inv;
                Chunk<CW>::store(y, base + c, o);
            }
        }
    }
}

template <int LPR, int NCH, int CW>
__global__ __launch_bounds__(kBlock) void softmax_bwd_kernel(half_t* dx, const half_t* y,
                                                             const half_t* dy, uint32_t rows,
                                                             uint32_t k) {
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l = lane % LPR;
    const int sub = lane / LPR;
    for (uint32_t r0 = blockIdx.x * (kWaves * RPW); r0 < rows; r0 += gridDim.x * (kWaves * RPW)) {
        const uint32_t row = r0 + wave * RPW + sub;
        const bool ok = row < rows;
        const size_t base = static_cast<size_t>(row) * k;
        typename Chunk<CW>::T ry[NCH], rd[NCH];
        {
            // Unconditional loads at indices clamped into the tensor (chunks
            // past the row end re-read its last one, a cache hit), zeroed
            // afterwards: a load under a branch can get a wait of its own.
            const size_t cbase = static_cast<size_t>(ok ? row : rows - 1) * k;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                const size_t i = cbase + (c < k ? c : k - CW);
                ry[j] = Chunk<CW>::load(y, i);
                rd[j] = Chunk<CW>::load(dy, i);
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const bool in = ok && (l + j * LPR) * CW < k;
                ry[j] = in ? ry[j] : Chunk<CW>::fill(0.0f);
                rd[j] = in ? rd[j] : Chunk<CW>::fill(0.0f);
            }
        }
        float vy[NCH][CW], vd[NCH][CW];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            Chunk<CW>::widen(ry[j], vy[j]);
            Chunk<CW>::widen(rd[j], vd[j]);
        }
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int q = 0; q < CW; ++q) dot = fmaf(vy[j][q], vd[j][q], dot);
        dot = group_sum<LPR>(dot);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (l + j * LPR) * CW;
            if (ok && c < k) {
                float o[CW];
#pragma unroll
                for (int q = 0; q < CW; ++q) o[q] = vy[j][q] * (vd[j][q] - dot);
                Chunk<CW>::store(dx, base + c, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One row per 1024-thread block (rows longer than 4096)
// ---------------------------------------------------------------------------
constexpr int kBigBlock = 1024;
constexpr int kBigWaves = kBigBlock / kWave;

__device__ __forceinline__ float block_max(float v, float* red) {
    v = group_max<64>(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kBigWaves; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = group_sum<64>(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kBigWaves; ++w) r += red[w];
    __syncthreads();
    return r;
}

template <int NCH, bool MASKED>
__global__ __launch_bounds__(kBigBlock) void softmax_fwd_block_kernel(half_t* y, const half_t* x,
                                                                      uint32_t rows, uint32_t k,
                                                                      RowMask mask) {
    __shared__ float red[kBigWaves];
    for (uint32_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const uint32_t n = valid_keys<MASKED>(mask, row, k);
        const size_t base = static_cast<size_t>(row) * k;
        half8 raw[NCH];
        if constexpr (!MASKED) {
            // Every key valid: unconditional loads (past the row end: its last
            // vector again), then -inf there.
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
                raw[j] = Chunk<8>::load(x, base + (c < k ? c : k - 8));
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                raw[j] = (threadIdx.x + j * kBigBlock) * 8 < n ? raw[j] : Chunk<8>::fill(-INFINITY);
        } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j) raw[j] = Chunk<8>::fill(-INFINITY);
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
                if (c < n) raw[j] = Chunk<8>::load(x, base + c);
            }
        }
        float v[NCH][8];
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
            Chunk<8>::widen(raw[j], v[j]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (MASKED && c + q >= n) v[j][q] = -INFINITY;
                m = fmaxf(m, v[j][q]);
            }
        }
        m = block_max(m, red);
        if (!(m > -INFINITY)) m = 0.0f;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                v[j][q] = __builtin_amdgcn_exp2f((v[j][q] - m) * kLog2e);
                s += v[j][q];
            }
        s = block_sum(s, red);
        const float inv = s > 0.0f ? 1.0f / s : 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
            if (c < k) {
                float o[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) o[q] = v[j][q] * inv;
                Chunk<8>::store(y, base + c, o);
            }
        }
    }
}

template <int NCH>
__global__ __launch_bounds__(kBigBlock) void softmax_bwd_block_kernel(half_t* dx, const half_t* y,
                                                                      const half_t* dy,
                                                                      uint32_t rows, uint32_t k) {
    __shared__ float red[kBigWaves];
    for (uint32_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const size_t base = static_cast<size_t>(row) * k;
        half8 ry[NCH], rd[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j) ry[j] = rd[j] = Chunk<8>::fill(0.0f);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
            if (c < k) {
                ry[j] = Chunk<8>::load(y, base + c);
                rd[j] = Chunk<8>::load(dy, base + c);
            }
        }
        float vy[NCH][8], vd[NCH][8];
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            Chunk<8>::widen(ry[j], vy[j]);
            Chunk<8>::widen(rd[j], vd[j]);
#pragma unroll
            for (int q = 0; q < 8; ++q) dot = fmaf(vy[j][q], vd[j][q], dot);
        }
        dot = block_sum(dot, red);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (threadIdx.x + j * kBigBlock) * 8;
            if (c < k) {
                float o[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) o[q] = vy[j][q] * (vd[j][q] - dot);
                Chunk<8>::store(dx, base + c, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch-shape table
// ---------------------------------------------------------------------------
struct SmShape {
    int lpr, nch, cw;     // lpr == 0: block-per-row path with nch chunks of 8 per thread
    const char* name;
};

constexpr int64_t kMaxKLen = 65536;
constexpr int64_t kMaxKLenScalar = 1024;

bool sm_shape(int64_t k, bool vec, SmShape* s) {
    if (vec) {
        const int64_t nv = k / 8;
        if (nv <= 8) *s = {8, 1, 8, "lpr8_nch1_v8"};
        else if (nv <= 16) *s = {8, 2, 8, "lpr8_nch2_v8"};
        else if (nv <= 32) *s = {16, 2, 8, "lpr16_nch2_v8"};
        else if (nv <= 64) *s = {32, 2, 8, "lpr32_nch2_v8"};
        else if (nv <= 128) *s = {64, 2, 8, "lpr64_nch2_v8"};
        else if (nv <= 256) *s = {64, 4, 8, "lpr64_nch4_v8"};
        else if (nv <= 512) *s = {64, 8, 8, "lpr64_nch8_v8"};
        else if (nv <= 1024) *s = {0, 1, 8, "block1024_nch1_v8"};
        else if (nv <= 2048) *s = {0, 2, 8, "block1024_nch2_v8"};
        else if (nv <= 4096) *s = {0, 4, 8, "block1024_nch4_v8"};
        else if (nv <= 8192) *s = {0, 8, 8, "block1024_nch8_v8"};
        else return false;
    } else {
        if (k <= 64) *s = {64, 1, 1, "lpr64_nch1_s"};
        else if (k <= 128) *s = {64, 2, 1, "lpr64_nch2_s"};
        else if (k <= 256) *s = {64, 4, 1, "lpr64_nch4_s"};
        else if (k <= 512) *s = {64, 8, 1, "lpr64_nch8_s"};
        else if (k <= 1024) *s = {64, 16, 1, "lpr64_nch16_s"};
        else return false;
    }
    return true;
}

// Rows of 72-128 keys take 8 lanes x 2 vectors; when that leaves fewer
// than 4096 waves (a quarter of the CUs' wave slots), 16 lanes x 1 vector
// instead: twice the waves, each row's loads spread over more lanes
// (BERT-base attention with 8 sequences of 128, 12288 rows: 3.17 against
// 3.35 us forward, 3.20 against 3.36 backward; with 32 sequences, 49152
// rows, 8 x 2 stays faster).
void few_rows_shape(int64_t rows, SmShape* s) {
    if (s->lpr == 8 && s->nch == 2 && rows * 8 < 4096 * int64_t{kWave}) *s = {16, 1, 8, "lpr16_nch1_v8"};
}

unsigned row_grid(int64_t rows, const SmShape& s) {
    const int64_t per_block = s.lpr ? kWaves * (kWave / s.lpr) : 1;
    const int64_t g = (rows + per_block - 1) / per_block;
    return static_cast<unsigned>(g < (1 << 20) ? g : (1 << 20));
}

int check_k(const char* name, int64_t k, bool vec, SmShape* s) {
    if (!sm_shape(k, vec, s)) {
        return fail(LS_ERR_UNSUPPORTED, "%s: k_len %lld exceeds %lld (%lld on the element-wise path)",
                    name, (long long)k, (long long)kMaxKLen, (long long)kMaxKLenScalar);
    }
    return LS_OK;
}

#define LS_SM_FWD(LPR, NCH, CW)                                                                 \
    do {                                                                                        \
        if (masked)                                                                             \
            softmax_fwd_kernel<LPR, NCH, CW, true><<<grid, kBlock, 0, st>>>(y16, x16, r32, k32, m); \
        else                                                                                    \
            softmax_fwd_kernel<LPR, NCH, CW, false><<<grid, kBlock, 0, st>>>(y16, x16, r32, k32, m); \
    } while (0)
#define LS_SM_FWD_BLOCK(NCH)                                                                    \
    do {                                                                                        \
        if (masked)                                                                             \
            softmax_fwd_block_kernel<NCH, true><<<grid, kBigBlock, 0, st>>>(y16, x16, r32, k32, m); \
        else                                                                                    \
            softmax_fwd_block_kernel<NCH, false><<<grid, kBigBlock, 0, st>>>(y16, x16, r32, k32, m); \
    } while (0)
#define LS_SM_BWD(LPR, NCH, CW)                                                                 \
    softmax_bwd_kernel<LPR, NCH, CW><<<grid, kBlock, 0, st>>>(dx16, y16, dy16, r32, k32)
#define LS_SM_BWD_BLOCK(NCH) softmax_bwd_block_kernel<NCH><<<grid, kBigBlock, 0, st>>>(dx16, y16, dy16, r32, k32)

#define LS_SM_TABLE(M, MB)                                                                      \
    if (s.lpr == 0) {                                                                           \
        switch (s.nch) {                                                                        \
            case 1: MB(1); break;                                                               \
            case 2: MB(2); break;                                                               \
            case 4: MB(4); break;                                                               \
            default: MB(8); break;                                                              \
        }                                                                                       \
    } else if (s.cw == 8) {                                                                     \
        if (s.lpr == 8 && s.nch == 1) M(8, 1, 8);                                               \
        else if (s.lpr == 8) M(8, 2, 8);                                                        \
        else if (s.lpr == 16 && s.nch == 1) M(16, 1, 8);                                        \
        else if (s.lpr == 16) M(16, 2, 8);                                                      \
        else if (s.lpr == 32) M(32, 2, 8);                                                      \
        else if (s.nch == 2) M(64, 2, 8);                                                       \
        else if (s.nch == 4) M(64, 4, 8);                                                       \
        else M(64, 8, 8);                                                                       \
    } else {                                                                                    \
        switch (s.nch) {                                                                        \
            case 1: M(64, 1, 1); break;                                                         \
            case 2: M(64, 2, 1); break;                                                         \
            case 4: M(64, 4, 1); break;                                                         \
            case 8: M(64, 8, 1); break;                                                         \
            default: M(64, 16, 1); break;                                                       \
        }                                                                                       \
    }

}  // namespace
}  // namespace ls

extern "C" {

int ls_softmax_fwd(void* y, const void* x, int64_t batch, int64_t heads, int64_t q_len,
                   int64_t k_len, const int32_t* key_lengths, int causal, void* stream) {
    using namespace ls;
    const char* name = "ls_softmax_fwd";
    if (batch < 0 || heads < 0 || q_len < 0 || k_len < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (batch == 0 || heads == 0 || q_len == 0 || k_len == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (heads > INT32_MAX / q_len || batch > INT32_MAX / (heads * q_len))
        return fail(LS_ERR_SHAPE, "%s: batch * heads * q_len must be < 2^31", name);
    if (!y || !x) return fail(LS_ERR_NULL, "%s: null pointer", name);
    const int64_t rows = batch * heads * q_len;
    const bool vec = k_len % 8 == 0 && aligned16(y) && aligned16(x);
    SmShape s;
    int rc = check_k(name, k_len, vec, &s);
    if (rc != LS_OK) return rc;
    few_rows_shape(rows, &s);
    const bool masked = key_lengths != nullptr || causal != 0;
    RowMask m;
    m.key_len = key_lengths;
    m.causal = causal != 0;
    m.q_len = FastDiv(static_cast<uint32_t>(q_len));
    m.per_batch = FastDiv(static_cast<uint32_t>(heads * q_len));
    const unsigned grid = row_grid(rows, s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* y16 = static_cast<half_t*>(y);
    auto* x16 = static_cast<const half_t*>(x);
    const uint32_t r32 = static_cast<uint32_t>(rows), k32 = static_cast<uint32_t>(k_len);
    clear_hip_error();
    LS_SM_TABLE(LS_SM_FWD, LS_SM_FWD_BLOCK)
    char buf[96];
    snprintf(buf, sizeof(buf), "softmax_fwd/%s%s", s.name, masked ? "_masked" : "");
    set_dispatch(buf);
    return launch_status(name);
}

int ls_softmax_bwd(void* dx, const void* y, const void* dy, int64_t rows, int64_t k_len, void* stream) {
    using namespace ls;
    const char* name = "ls_softmax_bwd";
    if (rows < 0 || k_len < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (rows == 0 || k_len == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: rows must be < 2^31", name);   // 32-bit row loops
    if (!dx || !y || !dy) return fail(LS_ERR_NULL, "%s: null pointer", name);
    const bool vec = k_len % 8 == 0 && aligned16(dx) && aligned16(y) && aligned16(dy);
    SmShape s;
    int rc = check_k(name, k_len, vec, &s);
    if (rc != LS_OK) return rc;
    few_rows_shape(rows, &s);
    const unsigned grid = row_grid(rows, s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* dx16 = static_cast<half_t*>(dx);
    auto* y16 = static_cast<const half_t*>(y);
    auto* dy16 = static_cast<const half_t*>(dy);
    const uint32_t r32 = static_cast<uint32_t>(rows), k32 = static_cast<uint32_t>(k_len);
    clear_hip_error();
    LS_SM_TABLE(LS_SM_BWD, LS_SM_BWD_BLOCK)
    char buf[96];
    snprintf(buf, sizeof(buf), "softmax_bwd/%s", s.name);
    set_dispatch(buf);
    return launch_status(name);
}

}  // extern "C"
