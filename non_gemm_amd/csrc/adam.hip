// Mixed-precision Adam over one contiguous fp16 workspace, one launch per
// step ([L10] technique 3, slide 29; [LS2] sec. 2.3).
//
// Parameters and gradients live only in fp16; each lane widens 16 of them
// (four 8-byte accesses each) to fp32 in registers, updates the fp32 moments
// (four 16-byte accesses each), and writes the parameter back rounded to
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
        p[i] = to_half(pn);
        m[i] = mi;
        v[i] = vi;
    }
}

// Vector body and scalar tail in one launch.  Each wave updates kSpan
// consecutive parameters per iteration, in kGroups groups of 256: lane L
// takes the four parameters at 4L of every group, so every load and store
// instruction of the wave covers one contiguous run (512 bytes of fp16,
// 1 KiB of fp32), and a lane has 4 x 4 loads in flight.  (Eight consecutive
// parameters per lane made each fp32 moment access a 32-byte-strided half of
// a 2 KiB run: 1423 us at 350M parameters; two groups per lane 1362 us, four
// 1310 us, eight spill past the register budget.)  The last block also
// finishes the parameters after the last whole group of four.
constexpr int kGroups = 4;
constexpr uint32_t kSpan = 256 * kGroups;                   // parameters per wave and iteration

template <bool DECOUPLED>
__global__ __launch_bounds__(kBlock) void adam_kernel(half_t* p, const half_t* g, float* m, float* v,
                                                      uint64_t n, uint64_t n4, AdamArgs a) {
    constexpr uint32_t kWavesPerBlock = kBlock / kWave;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint64_t grid_waves = static_cast<uint64_t>(gridDim.x) * kWavesPerBlock;
    for (uint64_t w = static_cast<uint64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; w * kSpan < n4;
         w += grid_waves) {
        // Every byte is touched exactly once per step: non-temporal accesses
        // stream it past the caches.  All loads before the first wait.
        half4 pq[kGroups], gq[kGroups];
        float4v mq[kGroups], vq[kGroups];
        bool ok[kGroups];
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const uint64_t i = w * kSpan + 256u * q + 4u * lane;
            ok[q] = i < n4;                                 // n4 % 4 == 0: a group of four is whole or absent
            pq[q] = gq[q] = half4{};
            mq[q] = vq[q] = float4v{};
            if (ok[q]) {
                pq[q] = __builtin_nontemporal_load(reinterpret_cast<const half4*>(p + i));
                gq[q] = __builtin_nontemporal_load(reinterpret_cast<const half4*>(g + i));
                mq[q] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(m + i));
                vq[q] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(v + i));
            }
        }
#pragma unroll
        for (int q = 0; q < kGroups; ++q)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float mk = mq[q][k], vk = vq[q][k];
                pq[q][k] = to_half(adam_one<DECOUPLED>(static_cast<float>(pq[q][k]),
                                                                   static_cast<float>(gq[q][k]), mk, vk, a));
                mq[q][k] = mk;
                vq[q][k] = vk;
            }
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            const uint64_t i = w * kSpan + 256u * q + 4u * lane;
            if (ok[q]) {
                __builtin_nontemporal_store(pq[q], reinterpret_cast<half4*>(p + i));
                __builtin_nontemporal_store(mq[q], reinterpret_cast<float4v*>(m + i));
                __builtin_nontemporal_store(vq[q], reinterpret_cast<float4v*>(v + i));
            }
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        for (uint64_t i = n4 + threadIdx.x; i < n; i += kBlock) {
            float mi = m[i], vi = v[i];
            const float pn = adam_one<DECOUPLED>(static_cast<float>(p[i]), static_cast<float>(g[i]), mi, vi, a);
            p[i] = to_half(pn);
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
        // One block per span of 4 waves x kSpan parameters: a capped
        // grid-stride launch measured slower on 256 CUs, whose block dispatch
        // keeps up with this body.
        const uint64_t per_block = static_cast<uint64_t>(kBlock / kWave) * kSpan;
        uint64_t blocks = (n4 + per_block - 1) / per_block;
        const uint64_t cap = 1ull << 30;
        if (blocks > cap) blocks = cap;
        if (blocks == 0) blocks = 1;
        if (decoupled_wd)
            adam_kernel<true><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, n4, a);
        else
            adam_kernel<false><<<static_cast<unsigned>(blocks), kBlock, 0, st>>>(p16, g16, exp_avg, exp_avg_sq, un, n4, a);
        set_dispatch(decoupled_wd ? "adam/groups4x4_adamw" : "adam/groups4x4_l2");
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
