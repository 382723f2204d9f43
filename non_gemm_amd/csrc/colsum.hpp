// Deterministic column sums for backward kernels whose parameter gradient is
// the sum over rows of a gradient they produce row by row (a bias).
//
// Layout of the work: the columns are cut into segments of 512 (one 16-byte
// vector of 8 fp16 per lane of a wave); a block of 16 waves owns one segment
// and one group of rows, each wave walking every 16th row of the group.  Each
// lane adds its 8 columns in fp32 registers; colsum_block_fold() folds the 16
// waves through LDS in wave order and writes the block's partial row; then
// colsum_finalize_kernel adds the partial rows of every column in a fixed
// order.  The result does not depend on timing: it is bit-reproducible.
#pragma once

#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kCsWaves = 16;
constexpr int kCsBlock = kCsWaves * kWave;      // 1024 threads
constexpr int kSegVecs = kWave;                 // 64 vectors = 512 columns per segment
constexpr int kSegCols = kSegVecs * 8;
constexpr int kMaxGroups = 256;
constexpr int kTargetWaves = 8192;              // two 16-wave blocks per CU: full occupancy
constexpr int kMinRowsPerWave = 2;

// Row groups: as many as keep ~kTargetWaves waves busy, at most one per 32
// rows (every wave gets two rows: with a single row nothing overlaps the wait
// for it) and at most kMaxGroups.  A function of the shape only, so a
// workspace can be sized before the pointers are known.
inline uint32_t colsum_groups(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    const int64_t segs = (cols + kSegCols - 1) / kSegCols;
    int64_t g = (kTargetWaves + kCsWaves * segs - 1) / (kCsWaves * segs);
    const int64_t by_rows = (rows + kCsWaves * kMinRowsPerWave - 1) / (kCsWaves * kMinRowsPerWave);
    if (g > by_rows) g = by_rows;
    if (g > kMaxGroups) g = kMaxGroups;
    return static_cast<uint32_t>(g < 1 ? 1 : g);
}

inline size_t colsum_workspace_bytes(int64_t rows, int64_t cols) {
    return static_cast<size_t>(colsum_groups(rows, cols)) * static_cast<size_t>(cols) * sizeof(float);
}

// Called by all kCsBlock threads of a (segment = blockIdx.x, group =
// blockIdx.y) block: lane l of wave w holds the sums of columns
// 512*blockIdx.x + 8*l + (0..7) over the rows that wave visited.
__device__ __forceinline__ void colsum_block_fold(float* partial, const float acc[8], uint32_t cols) {
    __shared__ float4v fold[kCsWaves][2][kSegVecs];     // 32 KiB: [wave][half][lane]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    fold[wave][0][lane] = float4v{acc[0], acc[1], acc[2], acc[3]};
    fold[wave][1][lane] = float4v{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    if (threadIdx.x < kSegCols) {
        const int c = threadIdx.x;
        const int l = c >> 3, k = c & 7;
        const uint32_t col = blockIdx.x * kSegCols + c;
        if (col < cols) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < kCsWaves; ++w) t += fold[w][k >> 2][l][k & 3];
            partial[static_cast<size_t>(blockIdx.y) * cols + col] = t;
        }
    }
}

// out[c] = sum over the partial rows g = 0..ngroups-1 of partial[g][c]: 32
// thread slices per column (slice s takes rows s, s+32, ...), then the 32
// slice sums in order.  ngroups == 0 writes zeros.  Every load is issued
// at an index clamped into the buffer and masked after it arrives: under a
// per-lane condition the compiler waited for the first load before issuing
// the rest.  A block takes 32 columns,
// so each partial row is read in whole 128-byte lines; 1024 threads with 8
// loads each (fewer loads per thread, more threads in flight, than 16 x 16).
constexpr int kFinCols = 32;
constexpr int kFinSlices = 32;
constexpr int kFinLoads = kMaxGroups / kFinSlices;
static_assert(kFinSlices * kFinLoads >= kMaxGroups, "the loads of a thread cover every partial row");

__global__ __launch_bounds__(kFinCols * kFinSlices) void colsum_finalize_kernel(half_t* out, const float* partial,
                                                                             uint32_t ngroups, uint32_t cols) {
    __shared__ float sums[kFinSlices][kFinCols];
    const int cl = threadIdx.x % kFinCols, sl = threadIdx.x / kFinCols;
    const uint32_t c = blockIdx.x * kFinCols + cl;
    float v[kFinLoads];
    if (ngroups) {
        const uint32_t cc = c < cols ? c : cols - 1;
#pragma unroll
        for (int i = 0; i < kFinLoads; ++i) {
            const uint32_t g = sl + i * kFinSlices;
            v[i] = partial[static_cast<size_t>(g < ngroups ? g : ngroups - 1) * cols + cc];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kFinLoads; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kFinLoads; ++i) v[i] = (c < cols && sl + i * kFinSlices < ngroups) ? v[i] : 0.0f;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kFinLoads; ++i) a += v[i];
    sums[sl][cl] = a;
    __syncthreads();
    if (sl == 0 && c < cols) {
        float t = 0.0f;
#pragma unroll
        for (int s = 0; s < kFinSlices; ++s) t += sums[s][cl];
        out[c] = to_half(t);
    }
}

inline void colsum_finalize(half_t* out, const float* partial, uint32_t ngroups, uint32_t cols, hipStream_t s) {
    colsum_finalize_kernel<<<(cols + kFinCols - 1) / kFinCols, kFinCols * kFinSlices, 0, s>>>(out, partial,
                                                                                          ngroups, cols);
}

// Host check of a caller's workspace for a column sum over [rows, cols].
inline int colsum_check_workspace(const char* name, const void* workspace, size_t bytes, int64_t rows,
                                  int64_t cols) {
    const size_t need = colsum_workspace_bytes(rows, cols);
    if (!workspace) return fail(LS_ERR_NULL, "%s: null workspace", name);
    if (bytes < need) return fail(LS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", name, bytes, need);
    if (!aligned16(workspace)) return fail(LS_ERR_PARAM, "%s: workspace must be 16-byte aligned", name);
    return LS_OK;
}

}  // namespace
}  // namespace ls
