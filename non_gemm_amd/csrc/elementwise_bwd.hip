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
#include "colsum.hpp"

namespace ls {
namespace {

template <bool RELU>
__global__ __launch_bounds__(kCsBlock) void ew_bwd_vec_kernel(half8* dx, float* partial, const half8* dy,
                                                               const half8* out, uint32_t rows,
                                                               uint32_t nv, uint32_t rows_per_group,
                                                               Dropout d) {
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
    for (; r < r_end; r += kCsWaves) {
        const uint32_t rn = r + kCsWaves;
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

    colsum_block_fold(partial, acc, nv * 8u);
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
        dx[i] = to_half(o);
    }
    partial[static_cast<size_t>(blockIdx.y) * cols + c] = acc;
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
    clear_hip_error();
    if (rows == 0) {                                   // no rows: d_bias is zero
        colsum_finalize(static_cast<half_t*>(dbias), nullptr, 0, static_cast<uint32_t>(cols), s);
        set_dispatch(RELU ? "bias_relu_dropout_bwd/empty_rows" : "bias_dropout_residual_bwd/empty_rows");
        return launch_status(name);
    }
    if (!dx || !dy || (RELU && !out)) return fail(LS_ERR_NULL, "%s: null tensor pointer", name);
    if (int rc = colsum_check_workspace(name, workspace, workspace_bytes, rows, cols)) return rc;
    const uint32_t groups = colsum_groups(rows, cols);
    float* part = static_cast<float*>(workspace);
    const uint64_t rpg = (static_cast<uint64_t>(rows) + groups - 1) / groups;
    const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols);
    const bool vec = cols % 8 == 0 && aligned16(dx) && aligned16(dy) && (!RELU || aligned16(out)) &&
                     n / 8 < (1ull << 31);
    char buf[96];
    if (vec) {
        const uint32_t nv = static_cast<uint32_t>(cols / 8);
        const dim3 grid((nv + kSegVecs - 1) / kSegVecs, groups);
        ew_bwd_vec_kernel<RELU><<<grid, kCsBlock, 0, s>>>(static_cast<half8*>(dx), part,
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
    colsum_finalize(static_cast<half_t*>(dbias), part, groups, static_cast<uint32_t>(cols), s);
    set_dispatch(buf);
    return launch_status(name);
}

}  // namespace
}  // namespace ls

extern "C" {

size_t ls_elementwise_bwd_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0 || cols >= (1ll << 31) || rows >= (1ll << 31)) return 0;
    return ls::colsum_workspace_bytes(rows, cols);
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
