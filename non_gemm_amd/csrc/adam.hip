// Mixed-precision Adam over one contiguous fp16 workspace, one launch per
// step ([L10] technique 3, slide 29; [LS2] sec. 2.3).
//
// Parameters and gradients live only in fp16; each lane widens 8 of them
// (one 16-byte access each) to fp32 in registers, updates the fp32 moments
// (two 16-byte accesses each), and writes the parameter back rounded to
// fp16.  Per parameter: 12 bytes read, 10 written.  Because the whole model
// sits in one workspace, the update is a single grid-stride kernel instead
// of one small kernel per parameter tensor.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;

struct AdamArgs {
    float lr, beta1, beta2, one_minus_beta1, one_minus_beta2, eps, wd;
    float inv_grad_scale;
    float inv_bc1;       // 1 / (1 - beta1^t)
    float inv_bc2;       // 1 / (1 - beta2^t)
};

template <bool DECOUPLED>
__device__ __forceinline__ float adam_one(float p, float g, float& m, float& v, const AdamArgs& a) {
    g *= a.inv_grad_scale;
    if (!DECOUPLED) g = fmaf(a.wd, p, g);
    m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
    v = fmaf(a.beta2, v, a.one_minus_beta2 * g * g);
    float u = (m * a.inv_bc1) / (sqrtf(v * a.inv_bc2) + a.eps);
    if (DECOUPLED) u = fmaf(a.wd, p, u);
    return fmaf(-a.lr, u, p);
}

// Element-wise path: the tail of the vector path (first == 8 * nvec), or the
// whole range when a pointer is not 16-byte aligned.
template <bool DECOUPLED>
__global__ __launch_bounds__(kBlock) void adam_scalar_kernel(half_t* p, const half_t* g, float* m,
                                                             float* v, uint64_t first, uint64_t n,
                                                             AdamArgs a) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = first + static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        float mi = m[i], vi = v[i];
        const float pn = adam_one<DECOUPLED>(static_cast<float>(p[i]), static_cast<float>(g[i]), mi, vi, a);
        p[i] = static_cast<half_t>(pn);
        m[i] = mi;
        v[i] = vi;
    }
}

// Vector body and scalar tail in one launch: blocks [0, nvec_blocks) run the
// vector loop, the last block also finishes the tail.
template <bool DECOUPLED>
__global__ __launch_bounds__(kBlock) void adam_kernel(half_t* p, const half_t* g, float* m, float* v,
                                                      uint64_t n, uint64_t nvec, AdamArgs a) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < nvec; i += stride) {
        half8* p8 = reinterpret_cast<half8*>(p);
        const half8* g8 = reinterpret_cast<const half8*>(g);
        float4v* m4 = reinterpret_cast<float4v*>(m);
        float4v* v4 = reinterpret_cast<float4v*>(v);
        // Every byte is touched exactly once per step: non-temporal accesses
        // stream it past the caches.
        const half8 pv = __builtin_nontemporal_load(p8 + i);
        const half8 gv = __builtin_nontemporal_load(g8 + i);
        float4v m0 = __builtin_nontemporal_load(m4 + 2 * i);
        float4v m1 = __builtin_nontemporal_load(m4 + 2 * i + 1);
        float4v v0 = __builtin_nontemporal_load(v4 + 2 * i);
        float4v v1 = __builtin_nontemporal_load(v4 + 2 * i + 1);
        float pf[8], gf[8], mf[8], vf[8];
        unpack8(pv, pf);
        unpack8(gv, gf);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            mf[k] = m0[k];
            mf[4 + k] = m1[k];
            vf[k] = v0[k];
            vf[4 + k] = v1[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) pf[k] = adam_one<DECOUPLED>(pf[k], gf[k], mf[k], vf[k], a);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m0[k] = mf[k];
            m1[k] = mf[4 + k];
            v0[k] = vf[k];
            v1[k] = vf[4 + k];
        }
        __builtin_nontemporal_store(pack8(pf), p8 + i);
        __builtin_nontemporal_store(m0, m4 + 2 * i);
        __builtin_nontemporal_store(m1, m4 + 2 * i + 1);
        __builtin_nontemporal_store(v0, v4 + 2 * i);
        __builtin_nontemporal_store(v1, v4 + 2 * i + 1);
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = nvec * 8 + threadIdx.x; i < n; i += kBlock) {
            float mi = m[i], vi = v[i];
            const float pn = adam_one<DECOUPLED>(static_cast<float>(p[i]), static_cast<float>(g[i]), mi, vi, a);
            p[i] = static_cast<half_t>(pn);
            m[i] = mi;
            v[i] = vi;
        }
    }
}

}  // namespace
}  // namespace ls

extern "C" int ls_adam_workspace_step(void* param, const void* grad, float* exp_avg,
                                      float* exp_avg_sq, int64_t n, float lr, float beta1,
                                      float beta2, float eps, float weight_decay, int64_t step,
                                      float grad_scale, int decoupled_wd, void* stream) {
    using namespace ls;
    const char* name = "ls_adam_workspace_step";
    if (n < 0) return fail(LS_ERR_SHAPE, "%s: negative n", name);
    if (!(lr >= 0.0f) || !host_finite(lr)) return fail(LS_ERR_PARAM, "%s: lr must be >= 0", name);
    if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
        return fail(LS_ERR_PARAM, "%s: betas must lie in [0, 1)", name);
    if (!(eps > 0.0f) || !host_finite(eps)) return fail(LS_ERR_PARAM, "%s: eps must be > 0", name);
    if (!(weight_decay >= 0.0f) || !host_finite(weight_decay))
        return fail(LS_ERR_PARAM, "%s: weight_decay must be >= 0", name);
    if (!(grad_scale > 0.0f) || !host_finite(grad_scale)) return fail(LS_ERR_PARAM, "%s: grad_scale must be > 0", name);
    if (step < 1) return fail(LS_ERR_PARAM, "%s: step is 1-based", name);
    if (n == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!param || !grad || !exp_avg || !exp_avg_sq) return fail(LS_ERR_NULL, "%s: null pointer", name);

    AdamArgs a;
    const double b1 = beta1, b2 = beta2, t = static_cast<double>(step);
    a.lr = lr;
    a.beta1 = beta1;
    a.beta2 = beta2;
    a.one_minus_beta1 = static_cast<float>(1.0 - b1);
    a.one_minus_beta2 = static_cast<float>(1.0 - b2);
    a.eps = eps;
    a.wd = weight_decay;
    a.inv_grad_scale = static_cast<float>(1.0 / grad_scale);
    a.inv_bc1 = static_cast<float>(1.0 / (1.0 - pow(b1, t)));
    a.inv_bc2 = static_cast<float>(1.0 / (1.0 - pow(b2, t)));

    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* p16 = static_cast<half_t*>(param);
    auto* g16 = static_cast<const half_t*>(grad);
    const bool vec = aligned16(param) && aligned16(grad) && aligned16(exp_avg) && aligned16(exp_avg_sq);
    const uint64_t un = static_cast<uint64_t>(n);
    clear_hip_error();
    if (vec) {
        const uint64_t nvec = un / 8;
        uint64_t blocks = (nvec + kBlock - 1) / kBlock;
        // One block per 256 vectors: a capped grid-stride launch measured
        // slower on 256 CUs, whose block dispatch keeps up with this body.
        const uint64_t cap = 1ull << 30;
        if (blocks > cap) blocks = cap;
        if (blocks == 0) blocks = 1;
        if (decoupled_wd)
            adam_kernel<true><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, nvec, a);
        else
            adam_kernel<false><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, nvec, a);
        set_dispatch(decoupled_wd ? "adam/vec8_adamw" : "adam/vec8_l2");
    } else {
        uint64_t blocks = (un + kBlock - 1) / kBlock;
        if (blocks > 65536) blocks = 65536;
        if (decoupled_wd)
            adam_scalar_kernel<true><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, 0, un, a);
        else
            adam_scalar_kernel<false><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, 0, un, a);
        set_dispatch(decoupled_wd ? "adam/scalar_adamw" : "adam/scalar_l2");
    }
    return launch_status(name);
}
