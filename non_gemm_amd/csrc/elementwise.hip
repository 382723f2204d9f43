// Fused elementwise kernels ([L10] technique 1, slide 12; [LS2] sec. 2.1.1):
//   bias + dropout + residual:  out = residual + keep * (x + bias) * scale
//   bias + ReLU + dropout:      out = keep * max(x + bias, 0) * scale
// plus the dropout-mask export used by tests.
//
// Each input byte is read once and each output byte written once; the
// dropout mask is regenerated from (seed, offset, element index) and never
// stored.  The vector path gives every lane whole 16-byte (8 x fp16)
// accesses, so one wave touches 1 KiB of contiguous memory per instruction,
// and one Philox call decides exactly the 8 elements of one access.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;
constexpr unsigned kGridCap = 8192;

template <bool RESID, bool RELU, bool DROP>
__device__ __forceinline__ void elementwise_vec8(half8* out, const half8 xv, const half8 bv, const half8 rv,
                                                 uint32_t v, const Dropout& d) {
    float a[8], b[8], r[8], f[8], o[8];
    unpack8(xv, a);
    unpack8(bv, b);
    if (RESID) unpack8(rv, r);
    if (DROP) {
        dropout_factors8(d, v, f);   // the vector index is the Philox call index
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k] = 1.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float t = a[k] + b[k];
        if (RELU) t = t < 0.0f ? 0.0f : t;   // NaN propagates
        o[k] = RESID ? fmaf(f[k], t, r[k]) : t * f[k];
    }
    // bias+dropout+residual's output is, in a layer, the LayerNorm's input
    // right after: a plain store leaves it in the caches (measured in the
    // BERT-base chain: 0.8 us per step faster than non-temporal).  The other
    // outputs are streamed.
    if (RESID) out[v] = pack8(o);
    else __builtin_nontemporal_store(pack8(o), out + v);
}

// One 16-byte vector per lane per iteration; the grid holds at most
// kGridCap blocks (four full-occupancy generations on 256 CUs), so larger
// tensors loop.  The loads of an iteration are issued before its Philox
// rounds, which run while they are in flight.
template <bool RESID, bool RELU, bool DROP>
__global__ __launch_bounds__(kBlock) void elementwise_vec_kernel(
    half8* out, const half8* x, const half8* bias, const half8* res, uint32_t nvec,
    FastDiv col_vecs, Dropout d) {
    const uint32_t stride = gridDim.x * kBlock;
    for (uint32_t v = blockIdx.x * kBlock + threadIdx.x; v < nvec; v += stride) {
        // Streamed operands: non-temporal loads and stores keep them from
        // displacing reusable lines (the bias) in the caches.
        const half8 bv = bias[col_vecs.mod(v)];
        const half8 xv = __builtin_nontemporal_load(x + v);
        half8 rv{};
        if (RESID) rv = __builtin_nontemporal_load(res + v);
        elementwise_vec8<RESID, RELU, DROP>(out, xv, bv, rv, v, d);
    }
}

// Element-wise fallback: any alignment, any column count, 64-bit indices.
template <bool RESID, bool RELU, bool DROP>
__global__ __launch_bounds__(kBlock) void elementwise_scalar_kernel(
    half_t* out, const half_t* x, const half_t* bias, const half_t* res, uint64_t n,
    uint64_t cols, Dropout d) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        float t = static_cast<float>(x[i]) + static_cast<float>(bias[i % cols]);
        if (RELU) t = t < 0.0f ? 0.0f : t;
        const float f = DROP ? dropout_factor1(d, i) : 1.0f;
        const float o = RESID ? fmaf(f, t, static_cast<float>(res[i])) : t * f;
        out[i] = to_half(o);
    }
}

__global__ __launch_bounds__(kBlock) void dropout_mask_kernel(uint8_t* keep, uint64_t n, Dropout d) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t call = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; call * 8 < n;
         call += stride) {
        float f[8];
        dropout_factors8(d, call, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint64_t i = call * 8 + j;
            if (i < n) keep[i] = (d.thr >= 65536u || f[j] == 0.0f) ? 0 : 1;
        }
    }
}

inline unsigned grid_for(uint64_t work, unsigned per_block, unsigned cap = 1u << 20) {
    const uint64_t g = (work + per_block - 1) / per_block;
    return static_cast<unsigned>(g < cap ? (g ? g : 1) : cap);
}

template <bool RESID, bool RELU>
int launch_elementwise(const char* name, void* out, const void* x, const void* bias,
                       const void* res, int64_t rows, int64_t cols, float p, uint64_t seed,
                       uint64_t offset, void* stream) {
    if (rows < 0 || cols < 0) return fail(LS_ERR_SHAPE, "%s: negative shape [%lld, %lld]", name,
                                          (long long)rows, (long long)cols);
    Dropout d;
    if (!make_dropout(p, seed, offset, &d))
        return fail(LS_ERR_PARAM, "%s: dropout probability %g outside [0, 1]", name, (double)p);
    if (rows == 0 || cols == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!out || !x || !bias || (RESID && !res))
        return fail(LS_ERR_NULL, "%s: null tensor pointer", name);
    if (rows > INT64_MAX / cols) return fail(LS_ERR_SHAPE, "%s: rows * cols overflows", name);
    const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols);
    const bool drop = d.thr != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();

    const bool vec = (cols % 8 == 0) && aligned16(out) && aligned16(x) && aligned16(bias) &&
                     (!RESID || aligned16(res)) && (n / 8) < (1ull << 31) &&
                     static_cast<uint64_t>(cols / 8) < (1ull << 31);
    if (vec) {
        const uint32_t nvec = static_cast<uint32_t>(n / 8);
        const FastDiv cv(static_cast<uint32_t>(cols / 8));
        // Below 2M vectors (32 MB of output) half the cap: measured 2 % faster on [4096, 3072]
        // and 0.3 us per BERT-base chain step; the larger Transformer-big shapes keep the full cap.
        const unsigned grid = grid_for(nvec, kBlock, nvec < (2u << 20) ? kGridCap / 2 : kGridCap);
        auto* o = static_cast<half8*>(out);
        auto* xv = static_cast<const half8*>(x);
        auto* bv = static_cast<const half8*>(bias);
        auto* rv = static_cast<const half8*>(res);
        if (drop)
            launch_kernel(elementwise_vec_kernel<RESID, RELU, true>, grid, kBlock, 0, s, o, xv, bv, rv, nvec, cv, d);
        else
            launch_kernel(elementwise_vec_kernel<RESID, RELU, false>, grid, kBlock, 0, s, o, xv, bv, rv, nvec, cv, d);
        set_dispatch(drop ? (RESID ? "bias_dropout_residual/vec8" : "bias_relu_dropout/vec8")
                          : (RESID ? "bias_dropout_residual/vec8_p0" : "bias_relu_dropout/vec8_p0"));
    } else {
        const unsigned grid = grid_for(n, kBlock, 65536);
        auto* o = static_cast<half_t*>(out);
        auto* xs = static_cast<const half_t*>(x);
        auto* bs = static_cast<const half_t*>(bias);
        auto* rs = static_cast<const half_t*>(res);
        if (drop)
            launch_kernel(elementwise_scalar_kernel<RESID, RELU, true>, grid, kBlock, 0, s, o, xs, bs, rs, n, cols, d);
        else
            launch_kernel(elementwise_scalar_kernel<RESID, RELU, false>, grid, kBlock, 0, s, o, xs, bs, rs, n, cols, d);
        set_dispatch(RESID ? "bias_dropout_residual/scalar" : "bias_relu_dropout/scalar");
    }
    return launch_status(name);
}

}  // namespace
}  // namespace ls

extern "C" {

int ls_bias_dropout_residual(void* out, const void* x, const void* bias, const void* residual,
                             int64_t rows, int64_t cols, float p, uint64_t seed, uint64_t offset,
                             void* stream) {
    return ls::launch_elementwise<true, false>("ls_bias_dropout_residual", out, x, bias, residual,
                                               rows, cols, p, seed, offset, stream);
}

int ls_bias_relu_dropout(void* out, const void* x, const void* bias, int64_t rows, int64_t cols,
                         float p, uint64_t seed, uint64_t offset, void* stream) {
    return ls::launch_elementwise<false, true>("ls_bias_relu_dropout", out, x, bias, nullptr, rows,
                                               cols, p, seed, offset, stream);
}

int ls_dropout_mask(uint8_t* keep, int64_t n, float p, uint64_t seed, uint64_t offset, void* stream) {
    using namespace ls;
    if (n < 0) return fail(LS_ERR_SHAPE, "ls_dropout_mask: negative n");
    Dropout d;
    if (!make_dropout(p, seed, offset, &d))
        return fail(LS_ERR_PARAM, "ls_dropout_mask: dropout probability %g outside [0, 1]", (double)p);
    if (n == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!keep) return fail(LS_ERR_NULL, "ls_dropout_mask: null pointer");
    clear_hip_error();
    const uint64_t calls = (static_cast<uint64_t>(n) + 7) / 8;
    dropout_mask_kernel<<<grid_for(calls, kBlock, 65536), kBlock, 0, static_cast<hipStream_t>(stream)>>>(
        keep, static_cast<uint64_t>(n), d);
    set_dispatch("dropout_mask");
    return launch_status("ls_dropout_mask");
}

}  // extern "C"
