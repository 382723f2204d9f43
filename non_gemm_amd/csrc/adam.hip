// Mixed-precision Adam over one contiguous fp16 workspace, one launch per
// step ([L10] technique 3, slide 29; [LS2] sec. 2.3).
//
// Parameters and gradients live only in fp16; each lane widens 8 of them
// (two 8-byte accesses each) to fp32 in registers, updates the fp32 moments
// (two 16-byte accesses each), and writes the parameter back rounded to
// fp16.  Per parameter: 12 bytes read, 10 written.  Because the whole model
// sits in one workspace, the update is a single grid-stride kernel instead
// of one small kernel per parameter tensor.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;
typedef half_t half4 __attribute__((ext_vector_type(4)));   // one 64-bit access

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

// Element-wise path: the whole range when a pointer is not 16-byte aligned.
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

// Vector body and scalar tail in one launch.  Each wave updates 512
// consecutive parameters per iteration: lane L takes parameters 4L..4L+3 and
// 256+4L..256+4L+3 of the span, so every load and store instruction of the
// wave covers one contiguous run (512 bytes of fp16, 1 KiB of fp32).  (With
// eight consecutive parameters per lane, each fp32 moment access was a
// 32-byte-strided half of a 2 KiB run, twice the cache lines per
// instruction: 1423 against 1375 us at 350M parameters.)  The last block
// also finishes the parameters after the last whole group of four.
template <bool DECOUPLED>
__global__ __launch_bounds__(kBlock) void adam_kernel(half_t* p, const half_t* g, float* m, float* v,
                                                      uint64_t n, uint64_t n4, AdamArgs a) {
    constexpr uint32_t kSpan = 8 * kWave;                 // parameters per wave and iteration
    constexpr uint32_t kWavesPerBlock = kBlock / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t grid_waves = static_cast<uint64_t>(gridDim.x) * kWavesPerBlock;
    for (uint64_t w = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; w * kSpan < n4;
         w += grid_waves) {
        const uint64_t q0 = w * kSpan + 4 * lane, q1 = q0 + kSpan / 2;
        const bool ok0 = q0 < n4, ok1 = q1 < n4;          // n4 % 4 == 0: a quad is whole or absent
        // Every byte is touched exactly once per step: non-temporal accesses
        // stream it past the caches.
        half4 p0{}, p1{}, g0{}, g1{};
        float4v m0{}, m1{}, v0{}, v1{};
        if (ok0) {
            p0 = __builtin_nontemporal_load(reinterpret_cast<const half4*>(p + q0));
            g0 = __builtin_nontemporal_load(reinterpret_cast<const half4*>(g + q0));
            m0 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(m + q0));
            v0 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(v + q0));
        }
        if (ok1) {
            p1 = __builtin_nontemporal_load(reinterpret_cast<const half4*>(p + q1));
            g1 = __builtin_nontemporal_load(reinterpret_cast<const half4*>(g + q1));
            m1 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(m + q1));
            v1 = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(v + q1));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float mk = m0[k], vk = v0[k];
            p0[k] = static_cast<half_t>(adam_one<DECOUPLED>(static_cast<float>(p0[k]), static_cast<float>(g0[k]),
                                                            mk, vk, a));
            m0[k] = mk;
            v0[k] = vk;
            mk = m1[k];
            vk = v1[k];
            p1[k] = static_cast<half_t>(adam_one<DECOUPLED>(static_cast<float>(p1[k]), static_cast<float>(g1[k]),
                                                            mk, vk, a));
            m1[k] = mk;
            v1[k] = vk;
        }
        if (ok0) {
            __builtin_nontemporal_store(p0, reinterpret_cast<half4*>(p + q0));
            __builtin_nontemporal_store(m0, reinterpret_cast<float4v*>(m + q0));
            __builtin_nontemporal_store(v0, reinterpret_cast<float4v*>(v + q0));
        }
        if (ok1) {
            __builtin_nontemporal_store(p1, reinterpret_cast<half4*>(p + q1));
            __builtin_nontemporal_store(m1, reinterpret_cast<float4v*>(m + q1));
            __builtin_nontemporal_store(v1, reinterpret_cast<float4v*>(v + q1));
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n4 + threadIdx.x; i < n; i += kBlock) {
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
        const uint64_t n4 = un / 4 * 4;
        // One block per span of 4 waves x 512 parameters: a capped
        // grid-stride launch measured slower on 256 CUs, whose block dispatch
        // keeps up with this body.
        const uint64_t per_block = static_cast<uint64_t>(kBlock / kWave) * 8 * kWave;
        uint64_t blocks = (n4 + per_block - 1) / per_block;
        const uint64_t cap = 1ull << 30;
        if (blocks > cap) blocks = cap;
        if (blocks == 0) blocks = 1;
        if (decoupled_wd)
            adam_kernel<true><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, n4, a);
        else
            adam_kernel<false><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, n4, a);
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
