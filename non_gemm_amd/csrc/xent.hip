// Cross-entropy criterion over vocabulary rows, forward and backward ([L10]
// technique 1, slide 12 names it among the fused reduce kernels; [LS2]
// sec. 2.1.3 defers its details to the slides).  With label smoothing eps
// (eps = 0: plain cross entropy) and one ignored target id:
//
//   lse_t  = log sum_j exp(x_tj)
//   loss_t = lse_t - (1 - eps) * x_t,y_t - eps * mean_j x_tj      (0 if y_t is ignored)
//   dx_tj  = g * (exp(x_tj - lse_t) - (1 - eps) * [j == y_t] - eps / V)   (0 if ignored)
//
// Forward: one block per row.  Each thread walks its 16-byte vectors of the
// row keeping a running (max m, sum l of exp(x - m), sum of x): the
// one-pass "online" form of the softmax normaliser ([CS336] sec. 6.2), so a
// row of any length is read exactly once.  The triples are merged across the
// wave by shuffles and across the waves in a fixed order, so lse is
// bit-reproducible; it is stored for the backward.
// Backward: no reduction left -- one 16-byte vector per lane over the flat
// [T, V] array, reading the row's saved lse and target.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kRowBlock = 512;
constexpr int kRowWaves = kRowBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;

struct Online {
    float m, l, sx;   // running max, sum of exp(x - m), sum of x
};

// exp2 on the hardware instruction (v_exp_f32): results below 2^-126 flush
// to zero, which cannot change a sum that already holds exp(0) = 1.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two partial states.  Commutative bit for bit (max, and a sum of the
// two rescaled terms), so every lane of a butterfly ends with the same state.
// A NaN in l stays NaN.  m = -inf means "nothing but -inf seen": l = 0.
__device__ __forceinline__ Online merge(const Online& a, const Online& b) {
    Online r;
    r.m = fmaxf(a.m, b.m);
    const float base = r.m > -INFINITY ? r.m : 0.0f;
    r.l = a.l * ex2((a.m - base) * kLog2e) + b.l * ex2((b.m - base) * kLog2e);
    r.sx = a.sx + b.sx;
    return r;
}

// Folds N new values into a thread's state: one rescale, then one
// exponential per value.  A NaN value makes its exponential, hence l, NaN
// for good; +inf gives exp(inf - inf) = NaN, as in the definition; -inf
// values add nothing.
template <int N>
__device__ __forceinline__ void absorb(Online& s, const float* x) {
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < N; ++k) cm = fmaxf(cm, x[k]);
    const float nm = fmaxf(s.m, cm);
    const float base = nm > -INFINITY ? nm : 0.0f;
    const float bl = base * kLog2e;
    float l = s.l * ex2(fmaf(s.m, kLog2e, -bl));
    float sx = s.sx;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        l += ex2(fmaf(x[k], kLog2e, -bl));
        sx += x[k];
    }
    s.m = nm;
    s.l = l;
    s.sx = sx;
}

__device__ __forceinline__ Online shfl_xor(const Online& s, int o) {
    return Online{__shfl_xor(s.m, o), __shfl_xor(s.l, o), __shfl_xor(s.sx, o)};
}

struct XentArgs {
    float one_minus_eps, eps_over_v, eps;
    int32_t ignore;
    uint32_t vocab;
};

// Block-wide merge of the threads' states and the row's outputs.
__device__ __forceinline__ void finish_row(Online s, uint32_t row, float* loss, float* lse, const half_t* xrow,
                                           const int32_t* targets, const XentArgs& a) {
    __shared__ Online part[kRowWaves];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) s = merge(s, shfl_xor(s, o));
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) part[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        Online t = part[0];
        for (int w = 1; w < kRowWaves; ++w) t = merge(t, part[w]);   // fixed order
        const float z = t.m + __logf(t.l);    // log-sum-exp
        const int32_t y = targets[row];
        float out;
        if (y == a.ignore) {
            out = 0.0f;
        } else if (y < 0 || static_cast<uint32_t>(y) >= a.vocab) {
            out = __builtin_nanf("");
        } else {
            const float xy = static_cast<float>(xrow[y]);
            out = z - a.one_minus_eps * xy - a.eps * (t.sx / static_cast<float>(a.vocab));
        }
        loss[row] = out;
        lse[row] = z;
    }
}

__global__ __launch_bounds__(kRowBlock) void xent_fwd_vec_kernel(float* loss, float* lse, const half8* logits,
                                                                 const int32_t* targets, uint32_t rows, uint32_t nv,
                                                                 XentArgs a) {
    const uint32_t row = blockIdx.x;
    const half8* x = logits + static_cast<size_t>(row) * nv;
    Online s{-INFINITY, 0.0f, 0.0f};
    uint32_t v = threadIdx.x;
    // Four vectors in flight per thread, then the remainder one at a time.
    for (; v + 3 * kRowBlock < nv; v += 4 * kRowBlock) {
        half8 h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) h[u] = __builtin_nontemporal_load(x + v + u * kRowBlock);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float f[8];
            unpack8(h[u], f);
            absorb<8>(s, f);
        }
    }
    for (; v < nv; v += kRowBlock) {
        float f[8];
        unpack8(__builtin_nontemporal_load(x + v), f);
        absorb<8>(s, f);
    }
    finish_row(s, row, loss, lse, reinterpret_cast<const half_t*>(x), targets, a);
}

// Element-wise path (V % 8 != 0 or unaligned logits): same state, one value at a time.
__global__ __launch_bounds__(kRowBlock) void xent_fwd_scalar_kernel(float* loss, float* lse, const half_t* logits,
                                                                    const int32_t* targets, uint32_t rows,
                                                                    XentArgs a) {
    const uint32_t row = blockIdx.x;
    const half_t* x = logits + static_cast<size_t>(row) * a.vocab;
    Online s{-INFINITY, 0.0f, 0.0f};
    for (uint32_t j = threadIdx.x; j < a.vocab; j += kRowBlock) {
        const float v = static_cast<float>(x[j]);
        absorb<1>(s, &v);
    }
    finish_row(s, row, loss, lse, x, targets, a);
}

// Backward: one 16-byte vector of 8 logits per lane.
constexpr int kBlock = 256;

__device__ __forceinline__ float xent_grad(float x, float z, uint32_t j, int32_t y, bool bad, float g,
                                           const XentArgs& a) {
    if (bad) return __builtin_nanf("");
    const float p = ex2((x - z) * kLog2e);
    const float t = (static_cast<int32_t>(j) == y ? a.one_minus_eps : 0.0f) + a.eps_over_v;
    return g * (p - t);
}

// Per element: one conversion, exp2 between two FMAs,
//   dx = g * 2^(x log2e - lse log2e) - g eps/V,
// and - g (1 - eps) once per row, in the one vector that holds the target.
// The gradient is computed whatever the target, then replaced for an
// ignored (0) or invalid (NaN) one: the logits are used on every path, so
// their load is issued with the target's and lse's, before one wait.
__global__ __launch_bounds__(kBlock) void xent_bwd_vec_kernel(half8* dx, const half8* logits, const int32_t* targets,
                                                              const float* lse, uint32_t nvec, FastDiv nv, float g,
                                                              XentArgs a) {
    const uint32_t v = blockIdx.x * kBlock + threadIdx.x;
    if (v >= nvec) return;
    const half8 h = __builtin_nontemporal_load(logits + v);
    const uint32_t row = nv.div(v);
    const uint32_t c0 = (v - row * nv.d) * 8;
    const int32_t y = targets[row];
    const float z = lse[row];
    float f[8], o[8];
    unpack8(h, f);
    const float zl = z * kLog2e;
    const float gb = -g * a.eps_over_v;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = fmaf(g, ex2(fmaf(f[k], kLog2e, -zl)), gb);
    const uint32_t d = static_cast<uint32_t>(y) - c0;
    if (d < 8u) {
        const float gt = g * a.one_minus_eps;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (d == static_cast<uint32_t>(k)) o[k] -= gt;
    }
    if (y == a.ignore || y < 0 || static_cast<uint32_t>(y) >= a.vocab) {
        const float r = y == a.ignore ? 0.0f : __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = r;
    }
    __builtin_nontemporal_store(pack8(o), dx + v);
}

__global__ __launch_bounds__(kBlock) void xent_bwd_scalar_kernel(half_t* dx, const half_t* logits,
                                                                 const int32_t* targets, const float* lse,
                                                                 uint64_t n, float g, XentArgs a) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const uint64_t row = i / a.vocab;
        const uint32_t j = static_cast<uint32_t>(i - row * a.vocab);
        const int32_t y = targets[row];
        float o = 0.0f;
        if (y != a.ignore) {
            const bool bad = y < 0 || static_cast<uint32_t>(y) >= a.vocab;
            o = xent_grad(static_cast<float>(logits[i]), lse[row], j, y, bad, g, a);
        }
        dx[i] = to_half(o);
    }
}

int xent_check(const char* name, int64_t rows, int64_t vocab, float eps) {
    if (rows < 0 || vocab < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (rows >= (1ll << 31) || vocab >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: shape too large", name);
    if (!(eps >= 0.0f && eps <= 1.0f)) return fail(LS_ERR_PARAM, "%s: smoothing must lie in [0, 1]", name);
    return LS_OK;
}

XentArgs xent_args(int64_t vocab, float eps, int32_t ignore) {
    XentArgs a;
    a.eps = eps;
    a.one_minus_eps = 1.0f - eps;
    a.eps_over_v = vocab > 0 ? static_cast<float>(static_cast<double>(eps) / static_cast<double>(vocab)) : 0.0f;
    a.ignore = ignore;
    a.vocab = static_cast<uint32_t>(vocab);
    return a;
}

}  // namespace
}  // namespace ls

extern "C" {

int ls_cross_entropy_fwd(float* loss, float* lse, const void* logits, const int32_t* targets, int64_t rows,
                         int64_t vocab, float smoothing, int32_t ignore_index, void* stream) {
    using namespace ls;
    const char* name = "ls_cross_entropy_fwd";
    if (int rc = xent_check(name, rows, vocab, smoothing)) return rc;
    if (rows == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (vocab == 0) return fail(LS_ERR_SHAPE, "%s: vocab must be >= 1", name);
    if (!loss || !lse || !logits || !targets) return fail(LS_ERR_NULL, "%s: null pointer", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const XentArgs a = xent_args(vocab, smoothing, ignore_index);
    clear_hip_error();
    const unsigned grid = static_cast<unsigned>(rows);
    if (vocab % 8 == 0 && aligned16(logits)) {
        xent_fwd_vec_kernel<<<grid, kRowBlock, 0, st>>>(loss, lse, static_cast<const half8*>(logits), targets,
                                                        static_cast<uint32_t>(rows),
                                                        static_cast<uint32_t>(vocab / 8), a);
        set_dispatch("cross_entropy_fwd/row_block512_v8");
    } else {
        xent_fwd_scalar_kernel<<<grid, kRowBlock, 0, st>>>(loss, lse, static_cast<const half_t*>(logits), targets,
                                                           static_cast<uint32_t>(rows), a);
        set_dispatch("cross_entropy_fwd/row_block512_scalar");
    }
    return launch_status(name);
}

int ls_cross_entropy_bwd(void* dlogits, const void* logits, const int32_t* targets, const float* lse, int64_t rows,
                         int64_t vocab, float smoothing, int32_t ignore_index, float grad_scale, void* stream) {
    using namespace ls;
    const char* name = "ls_cross_entropy_bwd";
    if (int rc = xent_check(name, rows, vocab, smoothing)) return rc;
    if (!host_finite(grad_scale)) return fail(LS_ERR_PARAM, "%s: grad_scale must be finite", name);
    if (rows == 0 || vocab == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!dlogits || !logits || !targets || !lse) return fail(LS_ERR_NULL, "%s: null pointer", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const XentArgs a = xent_args(vocab, smoothing, ignore_index);
    clear_hip_error();
    const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(vocab);
    if (vocab % 8 == 0 && aligned16(logits) && aligned16(dlogits) && n / 8 < (1ull << 31)) {
        const uint32_t nvec = static_cast<uint32_t>(n / 8);
        xent_bwd_vec_kernel<<<(nvec + kBlock - 1) / kBlock, kBlock, 0, st>>>(
            static_cast<half8*>(dlogits), static_cast<const half8*>(logits), targets, lse, nvec,
            FastDiv(static_cast<uint32_t>(vocab / 8)), grad_scale, a);
        set_dispatch("cross_entropy_bwd/vec8");
    } else {
        const uint64_t blocks = (n + kBlock - 1) / kBlock;
        xent_bwd_scalar_kernel<<<static_cast<unsigned>(blocks < 65536 ? blocks : 65536), kBlock, 0, st>>>(
            static_cast<half_t*>(dlogits), static_cast<const half_t*>(logits), targets, lse, n, grad_scale, a);
        set_dispatch("cross_entropy_bwd/scalar");
    }
    return launch_status(name);
}

}  // extern "C"
