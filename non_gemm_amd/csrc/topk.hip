// Beam-search top-k by hierarchical filtering (HARS, the inference half of
// [L10], "beam search" slides 45-54): instead of sorting all beam x V
// candidates of a step,
//   1. split a beam's candidates into k groups and take each group's max;
//   2. the smallest of those k maxima, R, is a value that at least k of the
//      beam's candidates reach, so the beam's k-th best is >= R;
//   3. keep only the candidates >= R and sort that short list.
// The candidates are c = log_prob[b, i, v] + beam_score[b, i] (one fp32 add),
// ranked by value, ties by the smaller flat index i * V + v.
//
// Two launches.  No beam contributes more than k candidates to the best k of
// its batch element, so each (batch element, beam) row gets a block of its
// own that runs the three steps above on that row and writes the row's best
// k, sorted, to the workspace; a second kernel sorts the beam x k survivors
// of each batch element and keeps the first k.  A row of up to 32768
// candidates is read once into registers (eight float4 per lane); each
// lane's values form group (lane mod k), so the group maxima are a reduction
// over lanes and waves.  Survivors go to an LDS list sorted by a bitonic
// network.  Should more than kCap candidates of a row survive (heavy ties),
// that block falls back to k exact passes of "largest rank below the
// previous pick" over the row, with the same result.
//
// Ordering: every fp32 value maps to an unsigned key that is monotone in the
// value (-0 < +0; every NaN is canonicalised to the largest key); a
// candidate's 64-bit rank is key << 32 | ~index, so larger is better and all
// ranks are distinct.  Rank 0 pads lists (below every real candidate).
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kTkBlock = 1024;
constexpr int kTkWaves = kTkBlock / kWave;
constexpr int kChunkVec = 8;                          // float4 per lane per chunk
constexpr int kChunk = kTkBlock * kChunkVec * 4;      // 32768 candidates per chunk
constexpr int kCap = 4096;                            // survivor list capacity (32 KiB of LDS)
constexpr int kMaxK = 1024;

__device__ __forceinline__ uint32_t key_of(float f) {
    if (f != f) return 0xFFFFFFFFu;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of key_of; the NaN key gives the default quiet NaN (payloads are not kept).
__device__ __forceinline__ float value_of(uint32_t k) {
    if (k == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t rank_of(uint32_t key, uint32_t idx) {
    return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~idx);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint64_t w = __shfl_xor(v, o);
        v = w > v ? w : v;
    }
    return v;
}

// Descending bitonic sort of list[0, n) (n a power of two) by all threads.
__device__ __forceinline__ void bitonic_desc(uint64_t* list, uint32_t n) {
    for (uint32_t size = 2; size <= n; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t t = threadIdx.x; t < n / 2; t += blockDim.x) {
                const uint32_t lo = 2 * stride * (t / stride) + (t % stride);
                const uint32_t hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = list[lo], c = list[hi];
                if ((a < c) == desc) {
                    list[lo] = c;
                    list[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

struct RowShared {
    uint64_t list[kCap];
    uint32_t gmax[kTkWaves][kWave];
    uint32_t group[kMaxK];
    uint64_t wbest[kTkWaves];
    uint32_t count;
    uint32_t thr;
};

// One (batch element, beam) row per block: its best k ranks, sorted, into
// best[row][0, k) (rank 0 where the row has fewer than k candidates).
// Eight waves per SIMD (two 1024-thread blocks per CU): 512 rows then run as
// one generation of blocks instead of two.  That caps the kernel at 64 VGPRs;
// about 18 of the row's values go to scratch once, after the threshold, and
// come back once (measured 26.1 -> 22.6 us on 128 x 4 rows of 32768; parking
// 16 of them in LDS, in the survivor list's space, instead measured 22.2
// against 21.7 us: the scratch round trip stays in the L2).
__global__ __launch_bounds__(kTkBlock, 8) void beam_row_topk_kernel(uint64_t* best, const float* lp,
                                                                 const float* beam_scores, uint32_t beam,
                                                                 uint32_t vocab, uint32_t k) {
    __shared__ RowShared sh;
    const uint32_t rowid = blockIdx.x;                 // b * beam + i
    const uint32_t i = rowid % beam;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const float* row = lp + static_cast<size_t>(rowid) * vocab;
    const float add = beam_scores ? beam_scores[rowid] : -0.0f;      // -0 + x == x exactly
    const bool vec = (vocab % 4 == 0) && ((reinterpret_cast<uintptr_t>(lp) & 15) == 0);
    const uint32_t nchunks = (vocab + kChunk - 1) / kChunk;
    if (tid == 0) sh.count = 0;

    auto elem = [&](uint32_t c, int u, int e) {
        return c * kChunk + (static_cast<uint32_t>(u) * kTkBlock + tid) * 4 + e;
    };
    // Candidate values of chunk c into x[] (slots past the row end are never
    // kept: keep() checks the index); returns the lane's largest key.  With
    // vocab % 4 == 0 a vector either lies inside the row or wholly past it.
    auto load_chunk = [&](uint32_t c, float x[kChunkVec * 4]) {
        // Every load of the chunk is issued before the first value is used.
        float4v q[kChunkVec];
#pragma unroll
        for (int u = 0; u < kChunkVec; ++u) q[u] = float4v{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (vec) {
#pragma unroll
            for (int u = 0; u < kChunkVec; ++u) {
                const uint32_t e0 = elem(c, u, 0);
                if (e0 < vocab) q[u] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(row + e0));
            }
        } else {
#pragma unroll
            for (int u = 0; u < kChunkVec; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (elem(c, u, e) < vocab) q[u][e] = row[elem(c, u, e)];
        }
        // The lane's largest value in the float domain (slots past the row
        // hold -inf): key_of(max) is at most the largest key (a NaN or a -0
        // against +0 can only lower it), so the group maxima and the
        // threshold drawn from them stay valid bounds, at one fmax per value
        // instead of a key each (measured 19.9 -> 18.5 us at 128 x 4 x 32768).
        float mf = -INFINITY;
#pragma unroll
        for (int u = 0; u < kChunkVec; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = q[u][e] + add;                // the one fp32 add of the definition
                x[u * 4 + e] = v;
                mf = fmaxf(mf, v);
            }
        return key_of(mf);
    };
    auto keep = [&](uint32_t c, const float x[kChunkVec * 4], uint32_t thr) {
        // A float pre-test first: every value whose key reaches thr also has
        // !(x < value_of(thr)) (NaN included), so the exact key test runs only
        // for the few that pass (21.7 -> 19.9 us at 128 x 4 x 32768).
        const float thr_f = thr ? value_of(thr) : -INFINITY;
#pragma unroll
        for (int u = 0; u < kChunkVec; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t v = elem(c, u, e);
                if (v < vocab && !(x[u * 4 + e] < thr_f) && key_of(x[u * 4 + e]) >= thr) {
                    const uint32_t key = key_of(x[u * 4 + e]);
                    const uint32_t slot = atomicAdd(&sh.count, 1u);
                    if (slot < kCap) sh.list[slot] = rank_of(key, i * vocab + v);
                }
            }
    };

    float x[kChunkVec * 4];
    uint32_t mk = 0;
    for (uint32_t c = 0; c < nchunks; ++c) mk = max(mk, load_chunk(c, x));

    // Steps 1-2: k groups (group = lane mod k) and the smallest group maximum.
    // A row shorter than k, or a group with no candidate, gives no bound (0).
    uint32_t thr = 0;
    if (vocab >= k) {
        if (k <= kWave && (kWave % k) == 0) {
            for (int o = kWave / 2; o >= static_cast<int>(k); o >>= 1)
                mk = max(mk, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mk), o)));
            sh.gmax[wave][lane] = mk;              // lane l now holds the wave's max of group l mod k
            __syncthreads();
            if (tid < static_cast<int>(k)) {
                uint32_t m = 0;
                for (int w = 0; w < kTkWaves; ++w) m = max(m, sh.gmax[w][tid]);
                sh.group[tid] = m;
            }
        } else {
            if (tid < static_cast<int>(k)) sh.group[tid] = 0;
            __syncthreads();
            atomicMax(&sh.group[static_cast<uint32_t>(tid) % k], mk);
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t m = 0xFFFFFFFFu;
            for (uint32_t q = lane; q < k; q += kWave) m = min(m, sh.group[q]);
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) m = min(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
            if (lane == 0) sh.thr = m;
        }
        __syncthreads();
        thr = sh.thr;
    }
    __syncthreads();

    // Step 3: keep the row's candidates at or above the threshold.
    if (nchunks == 1) {
        keep(0, x, thr);
    } else {
        for (uint32_t c = 0; c < nchunks; ++c) {
            load_chunk(c, x);
            keep(c, x, thr);
        }
    }
    __syncthreads();
    uint64_t* out = best + static_cast<size_t>(rowid) * k;
    const uint32_t count = sh.count;
    if (count <= static_cast<uint32_t>(kWave) && k <= static_cast<uint32_t>(kWave)) {
        // Short list: one wave sorts it in registers, no block barriers.
        if (wave == 0) {
            uint64_t key = static_cast<uint32_t>(lane) < count ? sh.list[lane] : 0;
            key = ~wave_sort_asc(~key, lane);          // descending; the padding ranks 0 come last
            if (static_cast<uint32_t>(lane) < k) out[lane] = key;
        }
        return;
    }
    if (count <= kCap) {
        uint32_t n = 2;
        while (n < count || n < k) n <<= 1;
        for (uint32_t s = count + tid; s < n; s += kTkBlock) sh.list[s] = 0;
        __syncthreads();
        bitonic_desc(sh.list, n);
        for (uint32_t j = tid; j < k; j += kTkBlock) out[j] = sh.list[j];
        return;
    }
    // Overflow: k exact passes over the row, each taking the largest rank below the last pick.
    uint64_t prev = ~0ull;
    for (uint32_t j = 0; j < k; ++j) {
        uint64_t m = 0;
        for (uint32_t v = tid; v < vocab; v += kTkBlock) {
            const uint64_t r = rank_of(key_of(row[v] + add), i * vocab + v);
            if (r < prev && r > m) m = r;
        }
        m = wave_max_u64(m);
        if (lane == 0) sh.wbest[wave] = m;
        __syncthreads();
        if (tid == 0) {
            uint64_t t = 0;
            for (int w = 0; w < kTkWaves; ++w) t = sh.wbest[w] > t ? sh.wbest[w] : t;
            sh.wbest[0] = t;
            out[j] = t;
        }
        __syncthreads();
        prev = sh.wbest[0];
        __syncthreads();
    }
}

// Per batch element: the beam x k row winners, sorted; the first k are the answer.
constexpr int kMergeBlock = 256;

__global__ __launch_bounds__(kMergeBlock) void beam_merge_kernel(float* top_scores, int32_t* top_ids,
                                                                 const uint64_t* best, uint32_t beam, uint32_t k) {
    __shared__ uint64_t list[kCap];
    const uint32_t b = blockIdx.x;
    const uint32_t m = beam * k;
    const uint64_t* src0 = best + static_cast<size_t>(b) * m;
    if (m <= static_cast<uint32_t>(kWave)) {          // one wave, in registers
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            uint64_t key = static_cast<uint32_t>(lane) < m ? src0[lane] : 0;
            key = ~wave_sort_asc(~key, lane);
            if (static_cast<uint32_t>(lane) < k) {
                top_scores[static_cast<size_t>(b) * k + lane] = value_of(static_cast<uint32_t>(key >> 32));
                top_ids[static_cast<size_t>(b) * k + lane] = static_cast<int32_t>(~static_cast<uint32_t>(key));
            }
        }
        return;
    }
    uint32_t n = 2;
    while (n < m) n <<= 1;
    const uint64_t* src = best + static_cast<size_t>(b) * m;
    for (uint32_t s = threadIdx.x; s < n; s += kMergeBlock) list[s] = s < m ? src[s] : 0;
    __syncthreads();
    bitonic_desc(list, n);
    for (uint32_t j = threadIdx.x; j < k; j += kMergeBlock) {
        const uint64_t r = list[j];
        top_scores[static_cast<size_t>(b) * k + j] = value_of(static_cast<uint32_t>(r >> 32));
        top_ids[static_cast<size_t>(b) * k + j] = static_cast<int32_t>(~static_cast<uint32_t>(r));
    }
}

int topk_check(const char* name, int64_t batch, int64_t beam, int64_t vocab, int64_t k) {
    if (batch < 0 || beam < 0 || vocab < 0 || k < 0) return fail(LS_ERR_SHAPE, "%s: negative size", name);
    if (batch == 0 || k == 0) return LS_OK;
    if (k > kMaxK) return fail(LS_ERR_UNSUPPORTED, "%s: k = %lld > %d", name, (long long)k, kMaxK);
    if (beam == 0 || vocab == 0 || beam > (1ll << 31) / vocab || k > beam * vocab)
        return fail(LS_ERR_SHAPE, "%s: need 1 <= k <= beam * vocab < 2^31", name);
    if (beam * k > kCap)
        return fail(LS_ERR_UNSUPPORTED, "%s: beam * k = %lld > %d", name, (long long)(beam * k), kCap);
    if (batch >= (1ll << 31) / beam) return fail(LS_ERR_SHAPE, "%s: batch * beam too large", name);
    return LS_OK;
}

}  // namespace
}  // namespace ls

extern "C" {

size_t ls_beam_topk_workspace_bytes(int64_t batch, int64_t beam, int64_t k) {
    if (batch <= 0 || beam <= 0 || k <= 0 || k > ls::kMaxK || beam * k > ls::kCap) return 0;
    return static_cast<size_t>(batch) * static_cast<size_t>(beam) * static_cast<size_t>(k) * sizeof(uint64_t);
}

int ls_beam_topk(float* top_scores, int32_t* top_ids, const float* log_probs, const float* beam_scores,
                 int64_t batch, int64_t beam, int64_t vocab, int64_t k, void* workspace, size_t workspace_bytes,
                 void* stream) {
    using namespace ls;
    const char* name = "ls_beam_topk";
    if (int rc = topk_check(name, batch, beam, vocab, k)) return rc;
    if (batch == 0 || k == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!top_scores || !top_ids || !log_probs) return fail(LS_ERR_NULL, "%s: null pointer", name);
    const size_t need = ls_beam_topk_workspace_bytes(batch, beam, k);
    if (!workspace) return fail(LS_ERR_NULL, "%s: null workspace", name);
    if (workspace_bytes < need)
        return fail(LS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", name, workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 8)
        return fail(LS_ERR_PARAM, "%s: workspace must be 8-byte aligned", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* best = static_cast<uint64_t*>(workspace);
    clear_hip_error();
    beam_row_topk_kernel<<<static_cast<unsigned>(batch * beam), kTkBlock, 0, st>>>(
        best, log_probs, beam_scores, static_cast<uint32_t>(beam), static_cast<uint32_t>(vocab),
        static_cast<uint32_t>(k));
    int rc = launch_status(name);
    if (rc != LS_OK) return rc;
    // beam * k <= 64 winners are sorted by one wave in registers: a one-wave block.
    const unsigned merge_threads = beam * k <= kWave ? kWave : kMergeBlock;
    beam_merge_kernel<<<static_cast<unsigned>(batch), merge_threads, 0, st>>>(top_scores, top_ids, best,
                                                                          static_cast<uint32_t>(beam),
                                                                          static_cast<uint32_t>(k));
    set_dispatch("beam_topk/hars_rows_block1024_merge");
    return launch_status(name);
}

}  // extern "C"
