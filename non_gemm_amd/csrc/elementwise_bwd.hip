// Backward of the two fused elementwise operators ([L10] technique 1,
// slide 12; [LS2] sec. 2.1.1 fuses each operator in both directions):
//
//   bias + dropout + residual:  d_x = dy * keep * scale,  d_bias = sum_rows d_x
//                               (d_residual = dy: nothing to compute)
//   bias + ReLU + dropout:      d_x = dy * [out > 0] * scale,  d_bias = sum_rows d_x
//
// The first regenerates the forward's Philox mask from (seed, offset); the
// second needs no random numbers: with fp16 inputs and scale >= 1, out > 0
// exactly when the element was kept and x + bias > 0, so the forward output
// carries the whole mask.
//
// One pass over the rows writes d_x and accumulates d_bias.  A wave owns a
// segment of 512 columns (one 16-byte vector of 8 per lane) and walks rows
// of its block's row group with the next row's loads in flight; the lanes
// keep fp32 column sums of the unrounded d_x in registers.  The 16 waves of a
// block fold their sums through LDS in wave order, the block writes one
// partial row, and a second kernel sums the partial rows column by column in
// a fixed order, so d_bias is bit-reproducible.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kWavesPerBlock = 16;
constexpr int kBwdBlock = kWavesPerBlock * kWave;      // 1024 threads
constexpr int kSegVecs = kWave;                        // 64 vectors = 512 columns per segment
constexpr int kSegCols = kSegVecs * 8;
constexpr int kMaxGroups = 256;
constexpr int kTargetWaves = 6144;                     // ~24 per CU: enough loads in flight

// Row groups: as many as keep ~kTargetWaves waves busy, at most one per 16
// rows (every wave gets a row) and at most kMaxGroups (the finalisation reads
// at most 16 partial rows per thread).  Depends on the shape only, so the
// workspace size is known before the pointers are.
uint32_t bwd_groups(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    const int64_t segs = (cols + kSegCols - 1) / kSegCols;
    int64_t g = (kTargetWaves + kWavesPerBlock * segs - 1) / (kWavesPerBlock * segs);
    const int64_t by_rows = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    if (g > by_rows) g = by_rows;
    if (g > kMaxGroups) g = kMaxGroups;
    return static_cast<uint32_t>(g < 1 ? 1 : g);
}

template <bool RELU>
__global__ __launch_bounds__(kBwdBlock) void ew_bwd_vec_kernel(half8* dx, float* partial, const half8* dy,
                                                               const half8* out, uint32_t rows,
                                                               uint32_t nv, uint32_t rows_per_group,
                                                               Dropout d) {
    __shared__ float4v fold[kWavesPerBlock][2][kSegVecs];   // 32 KiB: [wave][half][lane]
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t cv = blockIdx.x * kSegVecs + lane;        // this lane's vector column
    const bool col_ok = cv < nv;
    const uint32_t r_begin = blockIdx.y * rows_per_group;
    const uint32_t r_end = min(rows, r_begin + rows_per_group);

    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;

    uint32_t r = r_begin + wave;
    half8 gy{}, go{};
    if (col_ok && r < r_end) {
        const size_t v = static_cast<size_t>(r) * nv + cv;
        gy = __builtin_nontemporal_load(dy + v);
        if (RELU) go = __builtin_nontemporal_load(out + v);
    }
    for (; r < r_end; r += kWavesPerBlock) {
        const uint32_t rn = r + kWavesPerBlock;
        half8 ny{}, no{};
        if (col_ok && rn < r_end) {                          // next row's loads first
            const size_t v = static_cast<size_t>(rn) * nv + cv;
            ny = __builtin_nontemporal_load(dy + v);
            if (RELU) no = __builtin_nontemporal_load(out + v);
        }
        if (col_ok) {
            const size_t v = static_cast<size_t>(r) * nv + cv;
            float g[8], f[8], o[8];
            unpack8(gy, g);
            if (RELU) {
                float y[8];
                unpack8(go, y);
#pragma unroll
                for (int k = 0; k < 8; ++k) f[k] = y[k] > 0.0f ? d.scale : 0.0f;
            } else {
                dropout_factors8(d, v, f);       // the vector index is the forward's Philox call index
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                o[k] = g[k] * f[k];
                acc[k] += o[k];
            }
            __builtin_nontemporal_store(pack8(o), dx + v);
        }
        gy = ny;
        go = no;
    }

    fold[wave][0][lane] = float4v{acc[0], acc[1], acc[2], acc[3]};
    fold[wave][1][lane] = float4v{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    // Thread t < 512 sums column t of the segment over the 16 waves in order.
    if (threadIdx.x < kSegCols) {
        const int c = threadIdx.x;
        const int l = c >> 3, k = c & 7;
        const uint32_t col = blockIdx.x * kSegCols + c;
        if (col < nv * 8u) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < kWavesPerBlock; ++w) t += fold[w][k >> 2][l][k & 3];
            partial[static_cast<size_t>(blockIdx.y) * nv * 8u + col] = t;
        }
    }
}

// Element-wise path (cols % 8 != 0 or unaligned tensors): thread = one column
// of one row group, walking its rows; 64-bit element indices.
template <bool RELU>
__global__ __launch_bounds__(256) void ew_bwd_scalar_kernel(half_t* dx, float* partial, const half_t* dy,
                                                            const half_t* out, uint64_t rows, uint64_t cols,
                                                            uint64_t rows_per_group, Dropout d) {
    const uint64_t c = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= cols) return;
    const uint64_t r_begin = static_cast<uint64_t>(blockIdx.y) * rows_per_group;
    const uint64_t r_end = rows < r_begin + rows_per_group ? rows : r_begin + rows_per_group;
    float acc = 0.0f;
    for (uint64_t r = r_begin; r < r_end; ++r) {
        const uint64_t i = r * cols + c;
        const float f = RELU ? (static_cast<float>(out[i]) > 0.0f ? d.scale : 0.0f) : dropout_factor1(d, i);
        const float o = static_cast<float>(dy[i]) * f;
        acc += o;
        dx[i] = static_cast<half_t>(o);
    }
    partial[static_cast<size_t>(blockIdx.y) * cols + c] = acc;
}

// d_bias[c] = sum over the partial rows g = 0..ngroups-1 of partial[g][c]:
// 16 thread slices per column (slice s takes rows s, s+16, ...), then the 16
// slice sums in order.  ngroups == 0 writes zeros (no rows).
constexpr int kFinCols = 16;
constexpr int kFinSlices = 16;
static_assert(kFinSlices * 16 >= kMaxGroups, "16 loads per thread cover every partial row");

__global__ __launch_bounds__(kFinCols * kFinSlices) void colsum_finalize_kernel(half_t* dbias, const float* partial,
                                                                             uint32_t ngroups, uint32_t cols) {
    __shared__ float sums[kFinSlices][kFinCols];
    const int cl = threadIdx.x % kFinCols, sl = threadIdx.x / kFinCols;
    const uint32_t c = blockIdx.x * kFinCols + cl;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t g = sl + i * kFinSlices;
        v[i] = (c < cols && g < ngroups) ? partial[static_cast<size_t>(g) * cols + c] : 0.0f;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a += v[i];
    sums[sl][cl] = a;
    __syncthreads();
    if (sl == 0 && c < cols) {
        float t = 0.0f;
#pragma unroll
        for (int s = 0; s < kFinSlices; ++s) t += sums[s][cl];
        dbias[c] = static_cast<half_t>(t);
    }
}

template <bool RELU>
int launch_bwd(const char* name, void* dx, void* dbias, const void* dy, const void* out, int64_t rows,
               int64_t cols, float p, uint64_t seed, uint64_t offset, void* workspace,
               size_t workspace_bytes, void* stream) {
    if (rows < 0 || cols < 0)
        return fail(LS_ERR_SHAPE, "%s: negative shape [%lld, %lld]", name, (long long)rows, (long long)cols);
    Dropout d;
    if (!make_dropout(p, seed, offset, &d))
        return fail(LS_ERR_PARAM, "%s: dropout probability %g outside [0, 1]", name, (double)p);
    if (cols == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!dbias) return fail(LS_ERR_NULL, "%s: null dbias", name);
    if (cols >= (1ll << 31) || rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: shape too large", name);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned fgrid = static_cast<unsigned>((cols + kFinCols - 1) / kFinCols);
    clear_hip_error();
    if (rows == 0) {                                   // no rows: d_bias is zero
        colsum_finalize_kernel<<<fgrid, kFinCols * kFinSlices, 0, s>>>(static_cast<half_t*>(dbias), nullptr, 0,
                                                                       static_cast<uint32_t>(cols));
        set_dispatch(RELU ? "bias_relu_dropout_bwd/empty_rows" : "bias_dropout_residual_bwd/empty_rows");
        return launch_status(name);
    }
    if (!dx || !dy || (RELU && !out)) return fail(LS_ERR_NULL, "%s: null tensor pointer", name);
    const uint32_t groups = bwd_groups(rows, cols);
    const size_t need = static_cast<size_t>(groups) * static_cast<size_t>(cols) * sizeof(float);
    if (!workspace) return fail(LS_ERR_NULL, "%s: null workspace", name);
    if (workspace_bytes < need)
        return fail(LS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu", name, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(LS_ERR_PARAM, "%s: workspace must be 16-byte aligned", name);
    float* part = static_cast<float*>(workspace);
    const uint64_t rpg = (static_cast<uint64_t>(rows) + groups - 1) / groups;
    const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols);
    const bool vec = cols % 8 == 0 && aligned16(dx) && aligned16(dy) && (!RELU || aligned16(out)) &&
                     n / 8 < (1ull << 31);
    char buf[96];
    if (vec) {
        const uint32_t nv = static_cast<uint32_t>(cols / 8);
        const dim3 grid((nv + kSegVecs - 1) / kSegVecs, groups);
        ew_bwd_vec_kernel<RELU><<<grid, kBwdBlock, 0, s>>>(static_cast<half8*>(dx), part,
                                                           static_cast<const half8*>(dy),
                                                           static_cast<const half8*>(out),
                                                           static_cast<uint32_t>(rows), nv,
                                                           static_cast<uint32_t>(rpg), d);
        snprintf(buf, sizeof(buf), "%s/seg512_w16_g%u", RELU ? "bias_relu_dropout_bwd" : "bias_dropout_residual_bwd",
                 groups);
    } else {
        const dim3 grid(static_cast<unsigned>((cols + 255) / 256), groups);
        ew_bwd_scalar_kernel<RELU><<<grid, 256, 0, s>>>(static_cast<half_t*>(dx), part,
                                                       static_cast<const half_t*>(dy),
                                                       static_cast<const half_t*>(out),
                                                       static_cast<uint64_t>(rows),
                                                       static_cast<uint64_t>(cols), rpg, d);
        snprintf(buf, sizeof(buf), "%s/scalar_g%u", RELU ? "bias_relu_dropout_bwd" : "bias_dropout_residual_bwd",
                 groups);
    }
    int rc = launch_status(name);
    if (rc != LS_OK) return rc;
    colsum_finalize_kernel<<<fgrid, kFinCols * kFinSlices, 0, s>>>(static_cast<half_t*>(dbias), part, groups,
                                                                   static_cast<uint32_t>(cols));
    set_dispatch(buf);
    return launch_status(name);
}

}  // namespace
}  // namespace ls

extern "C" {

size_t ls_elementwise_bwd_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0 || cols >= (1ll << 31) || rows >= (1ll << 31)) return 0;
    return static_cast<size_t>(ls::bwd_groups(rows, cols)) * static_cast<size_t>(cols) * sizeof(float);
}

int ls_bias_dropout_residual_bwd(void* dx, void* dbias, const void* dy, int64_t rows, int64_t cols, float p,
                                 uint64_t seed, uint64_t offset, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return ls::launch_bwd<false>("ls_bias_dropout_residual_bwd", dx, dbias, dy, nullptr, rows, cols, p, seed,
                                 offset, workspace, workspace_bytes, stream);
}

int ls_bias_relu_dropout_bwd(void* dx, void* dbias, const void* dy, const void* out, int64_t rows, int64_t cols,
                             float p, void* workspace, size_t workspace_bytes, void* stream) {
    return ls::launch_bwd<true>("ls_bias_relu_dropout_bwd", dx, dbias, dy, out, rows, cols, p, 0, 0, workspace,
                                workspace_bytes, stream);
}

}  // extern "C"
