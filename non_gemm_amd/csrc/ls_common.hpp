// Device and host helpers shared by the ls_mi355 kernels (gfx950, wave64).
//
// Nothing here is specific to one operator: fp16 vector types, the Philox
// dropout decision, wave-level reductions built from DPP and swizzle
// instructions, a multiply-shift division for index arithmetic, and the
// thread-local error / dispatch bookkeeping of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "ls_mi355.h"

namespace ls {

// ---------------------------------------------------------------------------
// Types
// ---------------------------------------------------------------------------
typedef _Float16 half_t;
typedef half_t half8 __attribute__((ext_vector_type(8)));    // one 128-bit access
typedef float float4v __attribute__((ext_vector_type(4)));   // one 128-bit access

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Host-side bookkeeping (defined in abi.hip)
// ---------------------------------------------------------------------------
int fail(int status, const char* fmt, ...);       // records ls_last_error, returns status
void set_dispatch(const char* name);
int launch_status(const char* what);              // LS_OK or LS_ERR_HIP after a launch
void clear_hip_error();

// Events armed by ls_time_next_launch() for the calling thread, consumed by
// the next launch that goes through launch_kernel().
bool take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Launches kernel<<<grid, block, lds, stream>>>(args...); if the calling
// thread armed a pair of timing events, the launch records them itself
// (hipExtLaunchKernel), so they bracket the kernel's execution and nothing
// else.
template <typename... KArgs, typename... Args>
void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args... args) {
    hipEvent_t start, stop;
    if (take_launch_events(&start, &stop))
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, start, stop, 0u,
                              static_cast<KArgs>(args)...);
    else
        kernel<<<grid, block, lds, stream>>>(static_cast<KArgs>(args)...);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool host_finite(float x) { return std::isfinite(x); }

// ---------------------------------------------------------------------------
// Dropout: Philox4x32-10 [SC11], one call decides 8 consecutive elements
// ---------------------------------------------------------------------------
constexpr int kDropoutBits = 16;
constexpr int kDecisionsPerCall = 128 / kDropoutBits;   // 8 == elements per half8

struct Dropout {
    uint32_t k0, k1;     // key = seed
    uint32_t s0, s1;     // counter words 2, 3 = offset (the dropout site)
    uint32_t thr;        // drop iff 16-bit field < thr; thr in [0, 65536]
    float scale;         // 1 / (1 - thr / 65536), 0 when thr == 65536
};

// Validates p and builds the kernel-side parameters.  Returns false if p is
// outside [0, 1] (NaN included).
inline bool make_dropout(float p, uint64_t seed, uint64_t offset, Dropout* d) {
    if (!(p >= 0.0f && p <= 1.0f)) return false;
    const double thr = static_cast<double>(p) * 65536.0;       // exact
    d->thr = static_cast<uint32_t>(thr);                        // floor (thr >= 0)
    d->k0 = static_cast<uint32_t>(seed);
    d->k1 = static_cast<uint32_t>(seed >> 32);
    d->s0 = static_cast<uint32_t>(offset);
    d->s1 = static_cast<uint32_t>(offset >> 32);
    d->scale = d->thr >= 65536u ? 0.0f
                                : static_cast<float>(1.0 / (1.0 - d->thr / 65536.0));
    return true;
}

// Ten rounds of the Philox4x32 bijection on (c0..c3) under key (k0, k1).
// The multipliers and Weyl key increments are the ones [SC11] gives for
// Philox4x32.  The key words are wave-uniform, so the compiler keeps the
// key schedule in scalar registers.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
        const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
        // Three-input XOR in one v_bitop3_b32 (truth table 0x96).
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
    }
}

// The four Philox output words of call number `call` (counter = (call, offset)).
__device__ __forceinline__ void dropout_words(const Dropout& d, uint64_t call, uint32_t w[4]) {
    uint32_t c0 = static_cast<uint32_t>(call), c1 = static_cast<uint32_t>(call >> 32);
    uint32_t c2 = d.s0, c3 = d.s1;
    philox4x32_10(c0, c1, c2, c3, d.k0, d.k1);
    w[0] = c0;
    w[1] = c1;
    w[2] = c2;
    w[3] = c3;
}

// Keep factors from one call's words: scale where kept, 0 where dropped.
// Field j is bits [16*(j%2), 16*(j%2)+16) of word j/2.
__device__ __forceinline__ void dropout_factors_from(const Dropout& d, const uint32_t w[4], float f[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t field = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        f[j] = field >= d.thr ? d.scale : 0.0f;
    }
}

// Keep factors for the 8 elements 8*call .. 8*call+7.
__device__ __forceinline__ void dropout_factors8(const Dropout& d, uint64_t call, float f[8]) {
    uint32_t w[4];
    dropout_words(d, call, w);
    dropout_factors_from(d, w, f);
}

// Keep factor of the single element with flat index i.
__device__ __forceinline__ float dropout_factor1(const Dropout& d, uint64_t i) {
    float f[8];
    dropout_factors8(d, i >> 3, f);
    float r = f[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) r = (static_cast<int>(i & 7) == j) ? f[j] : r;
    return r;
}

// ---------------------------------------------------------------------------
// Wave-level reductions over aligned groups of W lanes (W = 8, 16, 32, 64).
// Every lane of a group ends with the same, bit-identical result (each step
// adds a pair of partial results; IEEE addition and max are commutative).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float swz_xor16(float v) {
    // ds_swizzle bit-mask mode inside 32-lane halves: and 0x1F, or 0, xor 0x10.
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }

// v from lane (lane ^ m), m a power of two below 64 (a constant after
// unrolling): DPP for 1 and 2, ds_swizzle (no LDS access) for 4..16, and
// ds_bpermute only across the two 32-lane halves.
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v, uint32_t m) {
    const int x = static_cast<int>(v);
    switch (m) {
        case 1: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, kDppXor1, 0xF, 0xF, false));
        case 2: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, kDppXor2, 0xF, 0xF, false));
        case 4: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, 0x101F));
        case 8: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, 0x201F));
        case 16: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, 0x401F));
        default: return static_cast<uint32_t>(__shfl_xor(x, static_cast<int>(m)));
    }
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    if (W >= 16) v += dpp<kDppMirror>(v);
    if (W >= 32) v += swz_xor16(v);
    if (W >= 64) v += xor32(v);
    return v;
}

// v of the first lane of this lane's aligned group of W lanes: a scalar read
// of lane 0 for the whole wave, a ds_bpermute (no LDS access) for narrower
// groups.  Every lane of the wave must be active.
template <int W>
__device__ __forceinline__ float group_first(float v, int lane) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    if constexpr (W == kWave)
        return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
    else
        return __shfl(v, lane & ~(W - 1));
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    if (W >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
    if (W >= 32) v = fmaxf(v, swz_xor16(v));
    if (W >= 64) v = fmaxf(v, xor32(v));
    return v;
}

// 64-bit lane exchange, and an ascending bitonic sort of one 64-bit key per
// lane across the whole wave (lane 0 ends with the smallest key).
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = lane_xor_u32(static_cast<uint32_t>(v), static_cast<uint32_t>(m));
    const uint32_t hi = lane_xor_u32(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(m));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t key, int lane) {
#pragma unroll
    for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t other = shfl_xor_u64(key, j);
            const bool ascending = (lane & k) == 0;
            const bool lower = (lane & j) == 0;
            const uint64_t lo = key < other ? key : other;
            const uint64_t hi = key < other ? other : key;
            key = (lower == ascending) ? lo : hi;
        }
    }
    return key;
}

// ---------------------------------------------------------------------------
// Unsigned division by a runtime constant d (1 <= d < 2^31) for numerators
// n < 2^31: q = (mulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (Granlund & Montgomery, PLDI'94).
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d, m, s;
    FastDiv() : d(1), m(1), s(0) {}
    explicit FastDiv(uint32_t div) : d(div) {
        s = 0;
        while ((1ull << s) < div) ++s;
        m = static_cast<uint32_t>(((1ull << 32) * ((1ull << s) - div)) / div + 1);
    }
    __device__ __forceinline__ uint32_t div(uint32_t n) const {
        return (__umulhi(n, m) + n) >> s;
    }
    __device__ __forceinline__ uint32_t mod(uint32_t n) const { return n - div(n) * d; }
};

// ---------------------------------------------------------------------------
// fp16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ void unpack8(const half8 h, float f[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = static_cast<float>(h[j]);
}
// fp32 -> fp16, round to nearest even, always from the fp32 value: the
// empty asm statement hides the value's origin, so the compiler cannot fold
// the conversion into the fma that produced it (v_fma_mix*_f16 rounds the
// exact product-sum straight to fp16, which can differ by one ulp from
// rounding the fp32 result, and whether it is chosen varies between
// instantiations of the same source).
__device__ __forceinline__ half_t to_half(float v) {
    asm("" : "+v"(v));
    return static_cast<half_t>(v);
}
__device__ __forceinline__ half8 pack8(const float f[8]) {
    half8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = to_half(f[j]);
    return h;
}

}  // namespace ls
