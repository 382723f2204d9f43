// LayerNorm forward and backward ([L10] technique 2, slides 21-22).
//
// Forward: one fused reduction per row.  Each lane accumulates S1 = sum d
// and S2 = sum d^2 over its elements, d = x - K with K the row's first
// element; the two sums travel through the same DPP/swizzle reduction, so
// the row needs a single cross-lane pass instead of "mean first, then
// variance":  mean = K + S1/H, var = S2/H - (S1/H)^2 (clamped at 0).  The
// same kernel (FUSED) also forms z = residual + Dropout(x + bias) chunk by
// chunk, stores it, and normalises it from registers: the sub-layer output
// block in one launch.
//
// Backward: the two row sums A = sum gamma*dy and B = sum gamma*dy*xhat are
// likewise reduced together, then dx = rstd * (gamma*dy - A/H - xhat*B/H).
// dgamma / dbeta are column sums over all rows: every block keeps per-lane
// fp32 column accumulators in registers over the rows it owns, folds them
// across its waves in a fixed order through LDS, and writes one partial row
// per block; a second kernel sums the partial rows in a fixed order (for up
// to 16 LayerNorms in one launch), so the result is bit-reproducible.
//
// Rows are mapped to aligned groups of LPR lanes (LPR = 8..64), each lane
// holding NCH chunks of CW consecutive elements (CW = 8: one 16-byte access
// per chunk; CW = 1: the element-wise path for unaligned rows).  Chunk j of
// lane l starts at column (l + j*LPR)*CW, so at every j the LPR lanes of a
// row read one contiguous span.
#include <mutex>
#include <type_traits>

#include "ls_common.hpp"

namespace ls {
namespace {

// Forward blocks of 256 threads, or of 1024 when the rows give every CU a
// whole 1024-thread block: fewer workgroups to dispatch for the same rows
// (4096 x 768: 5.15 -> 4.70 us; 512 threads 5.01), but with fewer rows the
// larger blocks leave CUs idle (1024 x 768: 3.61 us at 256 threads, 4.19 at
// 1024).  The 1024-thread form exists while a lane's raw row, gamma and beta
// fit in ~48 registers (up to 4 16-byte chunks, or 16 elements on the
// element-wise path, which keeps one per register): at most ~105 VGPRs, no
// spills.
constexpr int kFwdSmall = 256;
constexpr int kFwdBig = 1024;
constexpr bool fwd_big_ok(int nch, int cw, bool fused) {
    // the fused form also holds the residual and bias chunks
    return fused ? (cw == 8 ? nch <= 2 : nch <= 8) : (cw == 8 ? nch <= 4 : nch <= 16);
}

template <int CW>
struct Chunk;

template <>
struct Chunk<8> {
    static __device__ __forceinline__ void load(const half_t* p, size_t i, float f[8]) {
        unpack8(*reinterpret_cast<const half8*>(p + i), f);
    }
    // Outputs (y, dx) are written once and not read again by this kernel:
    // non-temporal stores keep them from displacing the reused gamma / beta.
    static __device__ __forceinline__ void store(half_t* p, size_t i, const float f[8]) {
        __builtin_nontemporal_store(pack8(f), reinterpret_cast<half8*>(p + i));
    }
};

template <>
struct Chunk<1> {
    static __device__ __forceinline__ void load(const half_t* p, size_t i, float f[1]) {
        f[0] = static_cast<float>(p[i]);
    }
    static __device__ __forceinline__ void store(half_t* p, size_t i, const float f[1]) {
        p[i] = to_half(f[0]);
    }
};

// Raw 16-byte (or 2-byte) row chunks.  In the forward's vector path a
// conditional load goes into a register set that was zeroed beforehand, so
// no instruction writes those registers after the load and every load of a
// row stays in flight until the first arithmetic that needs it; the backward
// loads unconditionally at clamped indices instead (its row pass says why).
template <int CW>
struct Raw;
template <>
struct Raw<8> {
    using T = half8;
    // The backward's row data (dy, x) are read once: non-temporal loads
    // stream them past the caches.
    static __device__ __forceinline__ T load(const half_t* p, size_t i) {
        return __builtin_nontemporal_load(reinterpret_cast<const half8*>(p + i));
    }
    // Plain loads: gamma and beta (read by every block), and the forward's x,
    // which in a layer was just written by the kernel before it (measured in
    // the BERT-base chain: 0.3 us per step faster than non-temporal, though
    // 0.2 us slower on cold input).
    static __device__ __forceinline__ T load_cached(const half_t* p, size_t i) {
        return *reinterpret_cast<const half8*>(p + i);
    }
    static __device__ __forceinline__ T zero() { return half8{0, 0, 0, 0, 0, 0, 0, 0}; }
    static __device__ __forceinline__ void widen(const T& r, float f[8]) { unpack8(r, f); }
};
// One fp16 element per 32-bit register (zero-extended): fp16 values kept two
// to a register would need each load merged into its pair as it arrives, a
// wait per element.
template <>
struct Raw<1> {
    using T = uint32_t;
    static __device__ __forceinline__ T load(const half_t* p, size_t i) {
        return reinterpret_cast<const uint16_t*>(p)[i];
    }
    static __device__ __forceinline__ T load_cached(const half_t* p, size_t i) { return load(p, i); }
    static __device__ __forceinline__ T zero() { return 0u; }
    static __device__ __forceinline__ void widen(const T& r, float f[1]) {
        f[0] = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(r)));
    }
};
// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// The fused form's extra operands: the row to normalise is
// z = residual + keep * (x + bias) * scale, computed like the standalone
// bias+dropout+residual (one fma per element, so z is bit-identical to it),
// rounded to fp16 and stored (the backward reads it), and the stored value
// is what the statistics see.  z may alias x or residual: each lane reads
// its elements before it writes them.
struct FwdFuse {
    half_t* z;
    const half_t* bias;
    const half_t* residual;
    Dropout d;
};

template <int LPR, int NCH, int CW, int BT, bool FUSED>
__global__ __launch_bounds__(BT) void ln_fwd_kernel(half_t* y, float* mean, float* rstd,
                                                        const half_t* x, const half_t* gamma,
                                                        const half_t* beta, uint32_t rows,
                                                        uint32_t h, float eps, FwdFuse fz) {
    constexpr int RPW = kWave / LPR;
    constexpr int kWaves = BT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int l = lane % LPR;
    const int sub = lane / LPR;

    using R = Raw<CW>;
    const float hf = static_cast<float>(h);
    for (uint32_t r0 = blockIdx.x * (kWaves * RPW); r0 < rows; r0 += gridDim.x * (kWaves * RPW)) {
        const uint32_t row = r0 + wave * RPW + sub;
        const bool ok = row < rows;
        const size_t base = static_cast<size_t>(row) * h;
        // The row's chunks first, then gamma and beta (cache hits after the
        // first waves); one wait covers all of them.
        constexpr int NF = FUSED ? NCH : 1;
        typename R::T xr[NCH], gr[NCH], br[NCH], rr[NF], cr[NF];    // rr, cr: residual, bias
        if constexpr (CW == 1) {
            // Element-wise path: unconditional loads at indices clamped into
            // the tensor, out-of-range values zeroed afterwards (a load
            // under a branch gets its conversion moved into the branch, a
            // wait per element).
            // (The fused form loads gamma and beta only after z is formed,
            // below, so that x, residual, bias, gamma and beta are never all
            // held at once.)
            const size_t cbase = static_cast<size_t>(ok ? row : rows - 1) * h;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = l + j * LPR;
                const uint32_t cc = c < h ? c : h - 1;
                xr[j] = R::load_cached(x, cbase + cc);
                if constexpr (FUSED) {
                    rr[j] = R::load_cached(fz.residual, cbase + cc);
                    cr[j] = R::load_cached(fz.bias, cc);
                } else {
                    gr[j] = R::load_cached(gamma, cc);
                    br[j] = R::load_cached(beta, cc);
                }
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const bool in = ok && l + j * LPR < h;
                xr[j] = in ? xr[j] : R::zero();
                if constexpr (FUSED) {
                    rr[j] = in ? rr[j] : R::zero();
                    cr[j] = in ? cr[j] : R::zero();
                } else {
                    gr[j] = in ? gr[j] : R::zero();
                    br[j] = in ? br[j] : R::zero();
                }
            }
        } else if constexpr (LPR < kWave) {
            // Rows that share a wave: the row chunks are loaded unconditionally
            // at clamped indices (past the row's end a lane reads its last
            // vector, past the last row the last row; nothing out of range is
            // stored, and the shift step zeroes such lanes), so none of their
            // registers is zeroed or copied ahead of the loads (4096 x 768
            // fused: 6.18-6.21 against 6.26-6.45 us).  With one row per wave
            // (below) the same form cost registers, and occupancy, at
            // 8192 x 1024.
#pragma unroll
            for (int j = 0; j < NCH; ++j) gr[j] = br[j] = R::zero();
#pragma unroll
            for (int j = 0; j < NF; ++j) cr[j] = R::zero();
            const size_t cbase = static_cast<size_t>(ok ? row : rows - 1) * h;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                const uint32_t cc = c < h ? c : h - CW;
                if constexpr (FUSED) {
                    xr[j] = R::load(x, cbase + cc);
                    rr[j] = R::load(fz.residual, cbase + cc);
                } else {
                    xr[j] = R::load_cached(x, cbase + cc);
                }
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                if (ok && c < h) {
                    if constexpr (FUSED) cr[j] = R::load_cached(fz.bias, c);
                    gr[j] = R::load_cached(gamma, c);
                    br[j] = R::load_cached(beta, c);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j) xr[j] = gr[j] = br[j] = R::zero();
#pragma unroll
            for (int j = 0; j < NF; ++j) rr[j] = cr[j] = R::zero();
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                if (ok && c < h) {
                    if constexpr (FUSED) {
                        // the fused inputs are read once: streamed
                        xr[j] = R::load(x, base + c);
                        rr[j] = R::load(fz.residual, base + c);
                    } else {
                        xr[j] = R::load_cached(x, base + c);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                if (ok && c < h) {
                    if constexpr (FUSED) cr[j] = R::load_cached(fz.bias, c);
                    gr[j] = R::load_cached(gamma, c);
                    br[j] = R::load_cached(beta, c);
                }
            }
        }
        // The dropout words of every chunk, computed while the loads are in
        // flight (they depend on the element index only).  With p = 0 the
        // threshold is 0 and every field keeps its element at scale 1, so no
        // branch is needed.
        // (The element-wise path computes each element's factor where it is
        // used: holding a field per element would cost a register each.)
        uint32_t dw[CW == 8 ? NF : 1][4];
        if constexpr (FUSED && CW == 8) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint64_t i0 = static_cast<uint64_t>(row) * h + (l + j * LPR) * CW;   // flat index
                dropout_words(fz.d, i0 >> 3, dw[j]);                       // h % 8 == 0: one Philox call
            }
            // Keep the rounds here, ahead of the first wait for the loads: the
            // words pass through an empty asm statement (no instruction), so
            // the compiler cannot sink later chunks' rounds into the blocks
            // that use them, after the wait.
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(dw[j][q]));
        }
        float v[NCH][CW];
        if constexpr (FUSED) {
            // z = residual + keep * (x + bias) * scale, rounded to fp16 and
            // stored; the statistics and y use the stored value.
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                float a[CW], b[CW], r[CW], f[CW], o[CW];
                R::widen(xr[j], a);
                R::widen(cr[j], b);
                R::widen(rr[j], r);
                if constexpr (CW == 8) dropout_factors_from(fz.d, dw[j], f);
                else f[0] = dropout_factor1(fz.d, static_cast<uint64_t>(row) * h + c);
#pragma unroll
                for (int k = 0; k < CW; ++k) o[k] = fmaf(f[k], a[k] + b[k], r[k]);
                if constexpr (CW == 8) {
                    const half8 zh = pack8(o);
                    if (ok && c < h) __builtin_nontemporal_store(zh, reinterpret_cast<half8*>(fz.z + base + c));
                    unpack8(zh, v[j]);
                } else {
                    const half_t zh = to_half(o[0]);
                    if (ok && c < h) fz.z[base + c] = zh;
                    v[j][0] = static_cast<float>(zh);
                }
            }
            if constexpr (CW == 1) {
                // gamma and beta for the element-wise path (cache hits), at
                // clamped indices, zero outside the row
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const uint32_t c = l + j * LPR;
                    const uint32_t cc = c < h ? c : h - 1;
                    gr[j] = R::load_cached(gamma, cc);
                    br[j] = R::load_cached(beta, cc);
                }
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const bool in = ok && l + j * LPR < h;
                    gr[j] = in ? gr[j] : R::zero();
                    br[j] = in ? br[j] : R::zero();
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NCH; ++j) R::widen(xr[j], v[j]);
        }
        // The sums run over d = x - K with K the row's first element (held by
        // the group's first lane): mean = K + S1'/H, var = S2'/H - (S1'/H)^2.
        // Still one fused reduction, but the cancellation is between terms of
        // the size of the row's spread rather than of its mean (shifted data,
        // Chan, Golub & LeVeque 1983), so rows whose |mean| is large next to
        // their spread keep fp32 accuracy.
        // Lane slots past the end of the row hold zeros and must stay zero
        // after the shift.
        const float K = group_first<LPR>(v[0][0], lane);
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int k = 0; k < CW; ++k) {
                v[j][k] = (l + j * LPR) * CW < h ? v[j][k] - K : 0.0f;
                s1 += v[j][k];
                s2 = fmaf(v[j][k], v[j][k], s2);
            }
        s1 = group_sum<LPR>(s1);          // the one fused reduction: (S1', S2') together
        s2 = group_sum<LPR>(s2);
        const float md = s1 / hf;
        const float var = fmaxf(s2 / hf - md * md, 0.0f);
        const float rs = rsqrtf(var + eps);
        if (ok && l == 0) {
            mean[row] = K + md;
            rstd[row] = rs;
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (l + j * LPR) * CW;
            if (ok && c < h) {
                float o[CW];
                float g[CW], b[CW];
                R::widen(gr[j], g);
                R::widen(br[j], b);
#pragma unroll
                for (int k = 0; k < CW; ++k) o[k] = fmaf((v[j][k] - md) * rs, g[k], b[k]);
                Chunk<CW>::store(y, base + c, o);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Backward, row pass
// ---------------------------------------------------------------------------
// Blocks of 4..16 waves (sized so that ~one block per CU covers the rows);
// each wave walks its rows, every load of a row issued before the first
// wait.  (A prefetch of the next row into a second register set measured
// slower, also written to fit 16-wave blocks without spilling.)  Once a wave
// has accumulated its last row, its per-lane column accumulators are folded
// across the row groups inside the wave (shuffles) and parked in the wave's
// LDS slot; after a barrier the slots are summed in wave order, and the block
// writes its partial row [2h] = (dgamma part, dbeta part).  The grid never
// exceeds the number of row groups, so every block, and every wave in it,
// takes at least one pass of the row loop, and each wave parks exactly once.
// Nothing but address arithmetic comes before a row's loads: the loads are
// unconditional at clamped indices (out-of-range lanes and rows zeroed after
// they arrive, not before), 1/h comes from the host, and the accumulators
// start from the first row's terms instead of being zeroed.  Work ahead of
// the loads delays every wave on a SIMD: without it the kernel measured 9.85
// against 10.12 us at 4096 x 768 and 15.37 against 15.60 at 8192 x 1024.
// Waves per block by register budget: 16 when a lane holds <= 16 elements
// (<= 128 VGPRs), 8 up to 32 elements, 4 beyond (one wave per SIMD, up to 512
// VGPRs, so the largest rows do not spill); the wave slots of the column fold
// take at most 128 KiB of LDS.
// The element-wise path (CW = 1) holds every element of a row in a register
// of its own (up to 32 per lane), so it takes smaller blocks.
constexpr int bwd_max_threads(int nch, int cw) {
    return cw == 1 ? (nch <= 8 ? 1024 : (nch <= 16 ? 512 : 256))
                   : (nch * cw <= 16 ? 1024 : (nch * cw <= 32 ? 512 : 256));
}
template <int NCH, int CW>
struct BwdBounds {
    static constexpr int kMaxThreads = bwd_max_threads(NCH, CW);
};
constexpr size_t kBwdLdsBudget = 128 * 1024;
// Columns per tile of the partial rows (one 128-byte line of floats).
constexpr uint32_t kPartTile = 32;

template <int LPR, int NCH, int CW>
__global__ __launch_bounds__((BwdBounds<NCH, CW>::kMaxThreads)) void ln_bwd_kernel(half_t* dx, float* partial,
                                                                uint32_t* header, const half_t* dy,
                                                                const half_t* x, const half_t* gamma,
                                                                const float* mean, const float* rstd,
                                                                uint32_t rows, uint32_t h, uint32_t slots,
                                                                float inv_h) {
    // The partial-row count, for the finalisation (which may run as a
    // separate call).
    if (blockIdx.x == 0 && threadIdx.x == 0) header[0] = gridDim.x;
    // Element-wise rows of up to 2048 hold one register per element; longer
    // ones are read twice (kTwoPass).
    constexpr bool kTwoPass = CW == 1 && NCH > 32;
    using R = Raw<CW>;
    constexpr int RPW = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const int l = lane % LPR;
    const int sub = lane / LPR;
    extern __shared__ float lds[];     // [nwaves][2h]

    // Rows (and gamma) stay in their fp16 form and are widened chunk by
    // chunk, twice (sums, then dx), so the registers hold raw rows plus the
    // accumulators.  The first pass of the row loop assigns the accumulators
    // (0 + term, so every value matches a sum started from zero); the
    // two-pass path keeps its column sums in the wave's LDS slot instead.
    constexpr int NACC = kTwoPass ? 1 : NCH;
    float acc_g[NACC][CW], acc_b[NACC][CW];
    const uint32_t per_iter = static_cast<uint32_t>(nwaves) * RPW;
    const uint32_t stride = gridDim.x * per_iter;
    const uint32_t my = static_cast<uint32_t>(wave) * RPW + sub;

    // Loads of one row: raw fp16 chunks, gamma (a cache hit, loaded again
    // with every row: kept from before the row loop, the wait for it would
    // come before the row's loads are issued) and the saved statistics.
    typename R::T rdy[NCH], rx[NCH], gr[NCH];
    float mu = 0.0f, rs = 0.0f;
    // Every load is unconditional, at an index clamped into its tensor (past
    // the row's end a lane reads the row's last vector or element, past the
    // last row a wave reads the last row), and values out of range are zeroed
    // once they arrive: a load under a per-lane condition made the compiler
    // wait for it, and registers zeroed ahead of the loads delay every wave
    // on the SIMD.
    auto fetch = [&](uint32_t row) {
        const bool ok = row < rows;
        const uint32_t rc = ok ? row : rows - 1;
        const size_t base = static_cast<size_t>(rc) * h;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (l + j * LPR) * CW;
            const uint32_t cc = c < h ? c : h - CW;
            rdy[j] = R::load(dy, base + cc);
            rx[j] = R::load(x, base + cc);
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const uint32_t c = (l + j * LPR) * CW;
            gr[j] = R::load_cached(gamma, c < h ? c : h - CW);
        }
        mu = mean[rc];
        rs = rstd[rc];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const bool in = ok && (l + j * LPR) * CW < h;
            rdy[j] = in ? rdy[j] : R::zero();
            rx[j] = in ? rx[j] : R::zero();
            gr[j] = in ? gr[j] : R::zero();
        }
        mu = ok ? mu : 0.0f;
        rs = ok ? rs : 0.0f;
    };
    // Parks this wave's column sums in its LDS slot.  Called right after the
    // last row's accumulation, so the LDS writes overlap that row's dx work
    // (0.1 us per call and 0.3 us per BERT-base step faster than after it).
    auto park = [&]() {
        if constexpr (!kTwoPass) {
            // Fold the RPW row groups of this wave (lanes l, l+LPR, ... own the same columns).
#pragma unroll
            for (int j = 0; j < NCH; ++j)
#pragma unroll
                for (int k = 0; k < CW; ++k)
#pragma unroll
                    for (int o = LPR; o < kWave; o <<= 1) {
                        acc_g[j][k] += __shfl_xor(acc_g[j][k], o);
                        acc_b[j][k] += __shfl_xor(acc_b[j][k], o);
                    }
            // Every wave parks its column sums in its own LDS slot [wave][2h]; after
            // one barrier each thread sums whole columns over the slots in wave order
            // and writes the block's partial row.  The order is fixed, so the sums are.
            if (sub == 0) {
                float* mine = lds + static_cast<size_t>(wave) * 2 * h;
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const uint32_t c = (l + j * LPR) * CW;
                    if (c < h) {
                        if constexpr (CW == 8) {      // two 16-byte LDS stores per half
                            float4v* pg = reinterpret_cast<float4v*>(mine + c);
                            float4v* pb = reinterpret_cast<float4v*>(mine + h + c);
                            pg[0] = float4v{acc_g[j][0], acc_g[j][1], acc_g[j][2], acc_g[j][3]};
                            pg[1] = float4v{acc_g[j][4], acc_g[j][5], acc_g[j][6], acc_g[j][7]};
                            pb[0] = float4v{acc_b[j][0], acc_b[j][1], acc_b[j][2], acc_b[j][3]};
                            pb[1] = float4v{acc_b[j][4], acc_b[j][5], acc_b[j][6], acc_b[j][7]};
                        } else {
#pragma unroll
                            for (int k = 0; k < CW; ++k) {
                                mine[c + k] = acc_g[j][k];
                                mine[h + c + k] = acc_b[j][k];
                            }
                        }
                    }
                }
            }
        }
    };
    if constexpr (kTwoPass) {
        // Element-wise rows longer than 2048: each row is read twice, in
        // batches of kB elements per lane -- sums, then dx from the caches --
        // and the column sums live in the wave's LDS slot [dgamma | dbeta],
        // where lane l owns columns l, l + 64, ... (no other lane touches them).
        constexpr int kB = 32;                  // two batches per pass
        static_assert(NCH % kB == 0, "whole batches");
        static_assert(LPR == kWave, "one row per wave");
        float* mine = lds + static_cast<size_t>(wave) * 2 * h;
        for (uint32_t c = l; c < h; c += LPR) mine[c] = mine[h + c] = 0.0f;
        for (uint32_t r0 = blockIdx.x * per_iter; r0 < rows; r0 += stride) {
            const uint32_t row = r0 + my;
            const bool ok = row < rows;
            const uint32_t rc = ok ? row : rows - 1;
            const size_t cbase = static_cast<size_t>(rc) * h;
            float sa = 0.0f, sb = 0.0f;
            const float m0 = ok ? mean[rc] : 0.0f, s0 = ok ? rstd[rc] : 0.0f;
#pragma unroll 1
            for (int b0 = 0; b0 < NCH; b0 += kB) {
                uint32_t ud[kB], ux[kB], ug[kB];
#pragma unroll
                for (int i = 0; i < kB; ++i) {
                    const uint32_t c = l + (b0 + i) * LPR;
                    const uint32_t cc = c < h ? c : h - 1;
                    ud[i] = R::load_cached(dy, cbase + cc);
                    ux[i] = R::load_cached(x, cbase + cc);
                    ug[i] = R::load_cached(gamma, cc);
                }
#pragma unroll
                for (int i = 0; i < kB; ++i) {
                    const bool in = ok && l + (b0 + i) * LPR < h;
                    float fd, fx, fg;
                    R::widen(ud[i], &fd);
                    R::widen(ux[i], &fx);
                    R::widen(ug[i], &fg);
                    fd = in ? fd : 0.0f;
                    fx = in ? fx : 0.0f;
                    fg = in ? fg : 0.0f;
                    const float xh = (fx - m0) * s0;
                    const float gd = fg * fd;
                    sa += gd;
                    sb = fmaf(gd, xh, sb);
                    const uint32_t c = l + (b0 + i) * LPR;
                    if (in) {
                        mine[c] = fmaf(fd, xh, mine[c]);
                        mine[h + c] += fd;
                    }
                }
            }
            sa = group_sum<LPR>(sa);
            sb = group_sum<LPR>(sb);
            const float ca = sa * inv_h, cb = sb * inv_h;
            if (ok) {
#pragma unroll 1
                for (int b0 = 0; b0 < NCH; b0 += kB) {
                    uint32_t ud[kB], ux[kB], ug[kB];
#pragma unroll
                    for (int i = 0; i < kB; ++i) {
                        const uint32_t c = l + (b0 + i) * LPR;
                        const uint32_t cc = c < h ? c : h - 1;
                        ud[i] = R::load_cached(dy, cbase + cc);
                        ux[i] = R::load_cached(x, cbase + cc);
                        ug[i] = R::load_cached(gamma, cc);
                    }
#pragma unroll
                    for (int i = 0; i < kB; ++i) {
                        const uint32_t c = l + (b0 + i) * LPR;
                        if (c < h) {
                            float fd, fx, fg, o;
                            R::widen(ud[i], &fd);
                            R::widen(ux[i], &fx);
                            R::widen(ug[i], &fg);
                            o = s0 * (fg * fd - fmaf((fx - m0) * s0, cb, ca));
                            Chunk<1>::store(dx, cbase + c, &o);
                        }
                    }
                }
            }
        }
    } else {
    // One pass of the row loop; `first` (a compile-time flag) marks the
    // wave's first row, whose terms start the accumulators.
    auto row_pass = [&](uint32_t r0, auto first) {
        const uint32_t row = r0 + my;
        fetch(row);
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            float fd[CW], fx[CW], fg[CW];
            R::widen(rdy[j], fd);
            R::widen(rx[j], fx);
            R::widen(gr[j], fg);
#pragma unroll
            for (int k = 0; k < CW; ++k) {
                const float xh = (fx[k] - mu) * rs;
                const float gd = fg[k] * fd[k];
                sa += gd;
                sb = fmaf(gd, xh, sb);
                if constexpr (decltype(first)::value) {
                    acc_g[j][k] = fmaf(fd[k], xh, 0.0f);
                    acc_b[j][k] = 0.0f + fd[k];
                } else {
                    acc_g[j][k] = fmaf(fd[k], xh, acc_g[j][k]);
                    acc_b[j][k] += fd[k];
                }
            }
        }
        if (r0 + stride >= rows) park();  // the wave's last row: sums complete
        sa = group_sum<LPR>(sa);          // the two row sums, reduced together
        sb = group_sum<LPR>(sb);
        const float ca = sa * inv_h, cb = sb * inv_h;
        if (row < rows) {
            const size_t base = static_cast<size_t>(row) * h;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const uint32_t c = (l + j * LPR) * CW;
                if (c < h) {
                    float fd[CW], fx[CW], fg[CW], o[CW];
                    R::widen(rdy[j], fd);
                    R::widen(rx[j], fx);
                    R::widen(gr[j], fg);
#pragma unroll
                    for (int k = 0; k < CW; ++k)
                        o[k] = rs * (fg[k] * fd[k] - fmaf((fx[k] - mu) * rs, cb, ca));
                    Chunk<CW>::store(dx, base + c, o);
                }
            }
        }
    };
    uint32_t r0 = blockIdx.x * per_iter;
    row_pass(r0, std::integral_constant<bool, true>{});
    for (r0 += stride; r0 < rows; r0 += stride) row_pass(r0, std::integral_constant<bool, false>{});
    }
    __syncthreads();
    // The block's partial row, in tiles of kPartTile columns: column col of block b
    // at t0 * slots + b * wt + (col - t0), where t0 is the tile's first
    // column and wt its width (kPartTile, less for a ragged last tile), so tile t
    // holds the slots rows of its columns contiguously; slots = the partial
    // rows the workspace holds (>= gridDim.x), and the last tile ends at
    // slots * 2h.
    for (uint32_t col = threadIdx.x; col < 2 * h; col += blockDim.x) {
        float t = 0.0f;
        for (int w = 0; w < nwaves; ++w) t += lds[static_cast<size_t>(w) * 2 * h + col];
        const uint32_t t0 = col / kPartTile * kPartTile, wt = min(kPartTile, 2 * h - t0);
        partial[static_cast<size_t>(t0) * slots + static_cast<size_t>(blockIdx.x) * wt + (col - t0)] = t;
    }
}

// Column finalisation over the nblocks partial rows of 2h columns (dgamma
// then dbeta): column c is summed by 32 thread slices (slice s takes blocks
// s, s+32, ...), then the 32 slice sums in order.  nblocks <= 256, so every
// thread issues at most 8 independent loads (1024-thread blocks: measured
// 0.3-0.4 us per BERT-base step faster than 16 slices of 16 loads).  The
// partials are stored in tiles of kPartTile columns (see the row kernel's store),
// and a block takes one tile, a single contiguous run of memory (measured
// 9.43-9.44 against 9.54-9.55 us per [4096, 768] operator call with the
// partial rows stored whole, 2h floats apart).
constexpr int kFinCols = kPartTile;
constexpr int kFinSlices = 32;
constexpr unsigned kMaxBwdBlocks = 256;
constexpr int kFinLoads = kMaxBwdBlocks / kFinSlices;

// Finalisations of up to kFinMaxJobs LayerNorms in one launch (a layer's or
// a model's LayerNorms, whose parameter gradients wait for the optimizer):
// job j takes blocks [first_block[j], first_block[j + 1]).  A thread loads
// its partial rows up to max_blocks (the count the workspace is sized for,
// indices clamped into it) together with the workspace header, and only then
// drops the rows past the header's count (clamped to max_blocks, so a stale
// header cannot widen the sum): no load waits for the header.  max_blocks == 0
// (no rows) writes zeros without reading the workspace.
constexpr int kFinMaxJobs = 16;
struct FinJobs {
    uint32_t count;
    uint32_t first_block[kFinMaxJobs + 1];
    uint32_t h[kFinMaxJobs];
    uint32_t max_blocks[kFinMaxJobs];
    half_t* dgamma[kFinMaxJobs];
    half_t* dbeta[kFinMaxJobs];
    const uint32_t* header[kFinMaxJobs];
    const float* partial[kFinMaxJobs];
};

__global__ __launch_bounds__(kFinCols * kFinSlices) void ln_bwd_finalize_kernel(const FinJobs jobs) {
    __shared__ float sums[kFinSlices][kFinCols];
    uint32_t j = 0;                              // uniform over the block
    while (j + 1 < jobs.count && blockIdx.x >= jobs.first_block[j + 1]) ++j;
    const uint32_t h = jobs.h[j], max_blocks = jobs.max_blocks[j];
    const float* partial = jobs.partial[j];
    const int cl = threadIdx.x % kFinCols, sl = threadIdx.x / kFinCols;
    const uint32_t t0 = (blockIdx.x - jobs.first_block[j]) * kFinCols, c = t0 + cl;
    const uint32_t w = 2 * h;
    float v[kFinLoads];
    uint32_t nblocks = 0;
    if (max_blocks) {
        const uint32_t cc = c < w ? c : w - 1;
#pragma unroll
        for (int i = 0; i < kFinLoads; ++i) {
            const uint32_t b = sl + i * kFinSlices;
            v[i] = partial[static_cast<size_t>(t0) * max_blocks +
                           static_cast<size_t>(b < max_blocks ? b : max_blocks - 1) * min(kPartTile, w - t0) + (cc - t0)];
        }
        nblocks = min(jobs.header[j][0], max_blocks);
    } else {
#pragma unroll
        for (int i = 0; i < kFinLoads; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kFinLoads; ++i) v[i] = (c < w && sl + i * kFinSlices < nblocks) ? v[i] : 0.0f;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kFinLoads; ++i) a += v[i];
    sums[sl][cl] = a;
    __syncthreads();
    if (sl == 0 && c < w) {
        float t = 0.0f;
#pragma unroll
        for (int s = 0; s < kFinSlices; ++s) t += sums[s][cl];
        if (c < h) jobs.dgamma[j][c] = to_half(t);
        else jobs.dbeta[j][c - h] = to_half(t);
    }
}

// ---------------------------------------------------------------------------
// Launch-shape table: (LPR, NCH, CW) from the row length.
// ---------------------------------------------------------------------------
struct LnShape {
    int lpr, nch, cw;
    const char* name;
};

bool ln_shape(int64_t h, bool vec, LnShape* s) {
    if (vec) {
        const int64_t nv = h / 8;
        if (nv <= 8) *s = {8, 1, 8, "lpr8_nch1_v8"};
        else if (nv <= 16) *s = {16, 1, 8, "lpr16_nch1_v8"};
        else if (nv <= 32) *s = {16, 2, 8, "lpr16_nch2_v8"};
        else if (nv <= 64) *s = {32, 2, 8, "lpr32_nch2_v8"};
        else if (nv <= 128) *s = {64, 2, 8, "lpr64_nch2_v8"};
        else if (nv <= 256) *s = {64, 4, 8, "lpr64_nch4_v8"};
        else if (nv <= 512) *s = {64, 8, 8, "lpr64_nch8_v8"};
        else return false;
    } else {
        if (h <= 64) *s = {64, 1, 1, "lpr64_nch1_s"};
        else if (h <= 128) *s = {64, 2, 1, "lpr64_nch2_s"};
        else if (h <= 256) *s = {64, 4, 1, "lpr64_nch4_s"};
        else if (h <= 512) *s = {64, 8, 1, "lpr64_nch8_s"};
        else if (h <= 1024) *s = {64, 16, 1, "lpr64_nch16_s"};
        else if (h <= 2048) *s = {64, 32, 1, "lpr64_nch32_s"};
        else if (h <= 4096) *s = {64, 64, 1, "lpr64_nch64_s"};
        else return false;
    }
    return true;
}

constexpr int64_t kMaxHidden = 4096;
constexpr size_t kBwdHeaderBytes = 256;       // partial rows start 256 bytes in
inline unsigned bwd_max_blocks(int64_t rows) {
    return static_cast<unsigned>(rows < kMaxBwdBlocks ? rows : kMaxBwdBlocks);
}
constexpr int kNumCU = 256;

unsigned fwd_grid(int64_t rows, const LnShape& s, int threads) {
    const int64_t per_block = threads / kWave * (kWave / s.lpr);
    const int64_t g = (rows + per_block - 1) / per_block;
    return static_cast<unsigned>(g < (1 << 20) ? g : (1 << 20));
}

// 1024-thread blocks when the shape allows them and the rows fill every CU
// with one; 256 otherwise.  The fused form always takes 256 (measured
// 7.1 against 7.3 us at 4096 x 768, 14.6 against 15.0 at 8192 x 1024).
int fwd_threads(int64_t rows, const LnShape& s, bool fused) {
    const int64_t rows_per_big = kFwdBig / kWave * (kWave / s.lpr);
    return !fused && fwd_big_ok(s.nch, s.cw, fused) && rows >= kNumCU * rows_per_big ? kFwdBig : kFwdSmall;
}

template <int LPR, int NCH, int CW, bool FUSED>
void launch_ln_fwd(int threads, unsigned grid, hipStream_t st, half_t* y, float* mean, float* rstd,
                   const half_t* x, const half_t* g, const half_t* b, uint32_t rows, uint32_t h, float eps,
                   const FwdFuse& fz) {
    if constexpr (fwd_big_ok(NCH, CW, FUSED)) {
        if (threads == kFwdBig) {
            launch_kernel(ln_fwd_kernel<LPR, NCH, CW, kFwdBig, FUSED>, dim3(grid), dim3(kFwdBig), 0, st, y, mean,
                          rstd, x, g, b, rows, h, eps, fz);
            return;
        }
    }
    launch_kernel(ln_fwd_kernel<LPR, NCH, CW, kFwdSmall, FUSED>, dim3(grid), dim3(kFwdSmall), 0, st, y, mean, rstd,
                  x, g, b, rows, h, eps, fz);
}

// Backward launch: waves per block (a power of two, 4 up to the shape's
// register and LDS limits) so that about one block per CU covers every row,
// then the block count (at most 256).  (Blocks of fewer waves for few rows
// measured slower: each block adds a partial row of 2h floats.)
struct BwdLaunch {
    int waves;
    unsigned grid;
    size_t lds_bytes;
};

BwdLaunch bwd_launch(int64_t rows, int64_t h, const LnShape& s) {
    BwdLaunch b;
    const int64_t rpw = kWave / s.lpr;
    const int max_waves = bwd_max_threads(s.nch, s.cw) / kWave;
    const int64_t want = (rows + kNumCU * rpw - 1) / (kNumCU * rpw);   // waves per block for one pass
    b.waves = 4;
    while (b.waves < max_waves && b.waves < want &&
           static_cast<size_t>(2 * b.waves) * 2 * h * sizeof(float) <= kBwdLdsBudget)
        b.waves *= 2;
    const int64_t per_block = b.waves * rpw;
    const int64_t g = (rows + per_block - 1) / per_block;
    b.grid = static_cast<unsigned>(g < kMaxBwdBlocks ? g : kMaxBwdBlocks);
    b.lds_bytes = static_cast<size_t>(b.waves) * 2 * h * sizeof(float);
    return b;
}

#define LS_LN_FWD(LPR, NCH, CW) \
    launch_ln_fwd<LPR, NCH, CW, false>(threads, grid, st, y16, mean, rstd, x16, g16, b16, r32, h32, eps, fz)
#define LS_LN_FWD_FUSED(LPR, NCH, CW)                                                                 \
    do {                                                                                              \
        if constexpr (CW == 8 || NCH <= 32)                                                           \
            launch_ln_fwd<LPR, NCH, CW, true>(threads, grid, st, y16, mean, rstd, x16, g16, b16, r32, h32, eps, fz); \
    } while (0)
#define LS_LN_BWD(LPR, NCH, CW)                                                                 \
    do {                                                                                        \
        if (bl.lds_bytes > 65536 &&                                                             \
            hipFuncSetAttribute(reinterpret_cast<const void*>(&ln_bwd_kernel<LPR, NCH, CW>),   \
                                hipFuncAttributeMaxDynamicSharedMemorySize,                    \
                                static_cast<int>(bl.lds_bytes)) != hipSuccess)                  \
            return fail(LS_ERR_HIP, "%s: cannot reserve %zu bytes of LDS", name, bl.lds_bytes); \
        launch_kernel(ln_bwd_kernel<LPR, NCH, CW>, dim3(bl.grid), dim3(bl.waves * kWave),         \
                      bl.lds_bytes, st, dx16, part, hdr, dy16, x16, g16, mean, rstd, r32, h32, \
                      bwd_max_blocks(r32), 1.0f / static_cast<float>(h32));    \
    } while (0)

#define LS_LN_TABLE(M)                                                                          \
    if (s.cw == 8) {                                                                            \
        if (s.lpr == 8) M(8, 1, 8);                                                             \
        else if (s.lpr == 16 && s.nch == 1) M(16, 1, 8);                                        \
        else if (s.lpr == 16) M(16, 2, 8);                                                      \
        else if (s.lpr == 32 && s.nch == 3) M(32, 3, 8);                                        \
        else if (s.lpr == 32) M(32, 2, 8);                                                      \
        else if (s.nch == 2) M(64, 2, 8);                                                       \
        else if (s.nch == 4) M(64, 4, 8);                                                       \
        else M(64, 8, 8);                                                                       \
    } else {                                                                                    \
        switch (s.nch) {                                                                        \
            case 1: M(64, 1, 1); break;                                                         \
            case 2: M(64, 2, 1); break;                                                         \
            case 4: M(64, 4, 1); break;                                                         \
            case 8: M(64, 8, 1); break;                                                         \
            case 16: M(64, 16, 1); break;                                                       \
            case 32: M(64, 32, 1); break;                                                       \
            default: M(64, 64, 1); break;                                                       \
        }                                                                                       \
    }

// ---------------------------------------------------------------------------
// Allocation-free LayerNorm backward: the workspace (header + partial rows)
// lives in a file-scope device array, one copy per GPU, held until the
// process ends.  2 MiB of partial rows cover hidden <= 1024 at any row count
// (at most 256 partial rows of 2 * hidden floats), and wider rows while
// rows * 2 * hidden * 4 bytes fit.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = kBwdHeaderBytes + (size_t(2) << 20);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current (in host code the array's name is only a
// stand-in for the symbol, never passed to a kernel or a copy).
int scratch_for_current_device(const char* name, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(LS_ERR_HIP, "%s: hipGetDevice failed", name);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(LS_ERR_UNSUPPORTED, "%s: device %d beyond the %d supported", name, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(LS_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", name, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LS_OK;
}

// Checks one parameter-gradient finalisation (the arguments of
// ls_layernorm_bwd_params); `who` names the call, and the job, in messages.
int check_params_job(const char* who, const void* dgamma, const void* dbeta, int64_t rows, int64_t hidden,
                     const void* workspace, size_t workspace_bytes) {
    if (rows < 0 || hidden < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", who);
    if (hidden == 0) return LS_OK;                 // nothing to write
    if (hidden > kMaxHidden)
        return fail(LS_ERR_UNSUPPORTED, "%s: hidden %lld > %lld", who, (long long)hidden, (long long)kMaxHidden);
    if (rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: rows must be < 2^31", who);
    if (!dgamma || !dbeta) return fail(LS_ERR_NULL, "%s: null pointer", who);
    if (rows > 0) {
        if (!workspace) return fail(LS_ERR_NULL, "%s: null workspace", who);
        const size_t need = ls_layernorm_bwd_workspace_bytes(rows, hidden);
        if (workspace_bytes < need)
            return fail(LS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, workspace_bytes, need);
        if (!aligned16(workspace)) return fail(LS_ERR_PARAM, "%s: workspace must be 16-byte aligned", who);
    }
    return LS_OK;
}

// Launches the finalisation of checked jobs, kFinMaxJobs per launch (jobs
// with hidden == 0 have nothing to write and are skipped), records the
// dispatch and returns the number of launches.
int launch_params_jobs(int count, void* const* dgamma, void* const* dbeta, const int64_t* rows,
                        const int64_t* hidden, void* const* workspace, hipStream_t st) {
    clear_hip_error();
    int launches = 0, jobs_run = 0;
    FinJobs fj{};
    auto flush = [&]() {
        if (fj.count == 0) return;
        launch_kernel(ln_bwd_finalize_kernel, dim3(fj.first_block[fj.count]), dim3(kFinCols * kFinSlices), 0, st,
                      fj);
        ++launches;
        fj = FinJobs{};
    };
    for (int i = 0; i < count; ++i) {
        if (hidden[i] == 0) continue;
        const uint32_t k = fj.count;
        const auto* ws = static_cast<const char*>(workspace[i]);
        const bool has_rows = rows[i] > 0;
        fj.h[k] = static_cast<uint32_t>(hidden[i]);
        fj.max_blocks[k] = has_rows ? bwd_max_blocks(rows[i]) : 0u;
        fj.dgamma[k] = static_cast<half_t*>(dgamma[i]);
        fj.dbeta[k] = static_cast<half_t*>(dbeta[i]);
        // A job with no rows reads nothing: the kernel never dereferences these.
        fj.header[k] = has_rows ? reinterpret_cast<const uint32_t*>(ws) : nullptr;
        fj.partial[k] = has_rows ? reinterpret_cast<const float*>(ws + kBwdHeaderBytes) : nullptr;
        fj.first_block[k + 1] =
            fj.first_block[k] + static_cast<uint32_t>((2 * hidden[i] + kFinCols - 1) / kFinCols);
        fj.count = k + 1;
        ++jobs_run;
        if (fj.count == kFinMaxJobs) flush();
    }
    flush();
    char buf[96];
    if (jobs_run == 0) snprintf(buf, sizeof(buf), "empty");
    else snprintf(buf, sizeof(buf), "layernorm_bwd_params/fixed_order_jobs%d_launches%d", jobs_run, launches);
    set_dispatch(buf);
    return launches;
}

}  // namespace
}  // namespace ls

extern "C" {

int ls_layernorm_fwd(void* y, float* mean, float* rstd, const void* x, const void* gamma,
                     const void* beta, int64_t rows, int64_t hidden, float eps, void* stream) {
    using namespace ls;
    const char* name = "ls_layernorm_fwd";
    if (rows < 0 || hidden < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (!(eps > 0.0f) || !host_finite(eps)) return fail(LS_ERR_PARAM, "%s: eps must be > 0", name);
    if (rows == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (hidden == 0) return fail(LS_ERR_SHAPE, "%s: hidden must be >= 1", name);
    if (hidden > kMaxHidden)
        return fail(LS_ERR_UNSUPPORTED, "%s: hidden %lld > %lld", name, (long long)hidden, (long long)kMaxHidden);
    if (rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: rows must be < 2^31", name);   // 32-bit row loops
    if (!y || !mean || !rstd || !x || !gamma || !beta) return fail(LS_ERR_NULL, "%s: null pointer", name);
    const bool vec = hidden % 8 == 0 && aligned16(y) && aligned16(x) && aligned16(gamma) && aligned16(beta);
    LnShape s;
    ln_shape(hidden, vec, &s);
    const int threads = fwd_threads(rows, s, false);
    const unsigned grid = fwd_grid(rows, s, threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* y16 = static_cast<half_t*>(y);
    auto* x16 = static_cast<const half_t*>(x);
    auto* g16 = static_cast<const half_t*>(gamma);
    auto* b16 = static_cast<const half_t*>(beta);
    const uint32_t r32 = static_cast<uint32_t>(rows), h32 = static_cast<uint32_t>(hidden);
    const FwdFuse fz{};
    clear_hip_error();
    LS_LN_TABLE(LS_LN_FWD)
    char buf[96];
    snprintf(buf, sizeof(buf), "layernorm_fwd/%s_b%d", s.name, threads);
    set_dispatch(buf);
    return launch_status(name);
}

int ls_bias_dropout_residual_layernorm(void* z, void* y, float* mean, float* rstd, const void* x,
                                       const void* bias, const void* residual, const void* gamma,
                                       const void* beta, int64_t rows, int64_t hidden, float p, uint64_t seed,
                                       uint64_t offset, float eps, void* stream) {
    using namespace ls;
    const char* name = "ls_bias_dropout_residual_layernorm";
    if (rows < 0 || hidden < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (!(eps > 0.0f) || !host_finite(eps)) return fail(LS_ERR_PARAM, "%s: eps must be > 0", name);
    FwdFuse fz;
    if (!make_dropout(p, seed, offset, &fz.d))
        return fail(LS_ERR_PARAM, "%s: dropout probability %g outside [0, 1]", name, (double)p);
    if (rows == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (hidden == 0) return fail(LS_ERR_SHAPE, "%s: hidden must be >= 1", name);
    if (hidden > kMaxHidden)
        return fail(LS_ERR_UNSUPPORTED, "%s: hidden %lld > %lld", name, (long long)hidden, (long long)kMaxHidden);
    if (rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: rows must be < 2^31", name);   // 32-bit row loops
    if (!z || !y || !mean || !rstd || !x || !bias || !residual || !gamma || !beta)
        return fail(LS_ERR_NULL, "%s: null pointer", name);
    const bool vec = hidden % 8 == 0 && aligned16(z) && aligned16(y) && aligned16(x) && aligned16(bias) &&
                     aligned16(residual) && aligned16(gamma) && aligned16(beta);
    LnShape s;
    ln_shape(hidden, vec, &s);
    if (vec && hidden / 8 > 64 && hidden / 8 <= 96) {
        // 65-96 vectors per row: 32 lanes x 3 chunks, two rows per wave, every
        // lane busy (64 x 2 leaves half the lanes idle on the second chunk), and
        // each load of bias, gamma and beta serves both rows of the wave:
        // 7.2 -> 6.3 us at 4096 x 768.  (The standalone LayerNorm forward,
        // with two parameter arrays, measured slower this way: 4.33 against
        // 4.21 us; 32 x 4 at 1024 columns too: 14.9 against 14.7 us.)
        s = {32, 3, 8, "lpr32_nch3_v8"};
    }
    if (s.cw == 1 && s.nch > 32) {
        // Element-wise rows longer than 2048 do not fit the fused kernel's
        // registers (x, residual, bias and each element's dropout words):
        // the two standalone operators, one after the other, give the same
        // bits.
        int rc = ls_bias_dropout_residual(z, x, bias, residual, rows, hidden, p, seed, offset, stream);
        if (rc != LS_OK) return rc;
        rc = ls_layernorm_fwd(y, mean, rstd, z, gamma, beta, rows, hidden, eps, stream);
        if (rc != LS_OK) return rc;
        char buf[112];
        snprintf(buf, sizeof(buf), "bias_dropout_residual_layernorm/two_launches_%s", s.name);
        set_dispatch(buf);
        return LS_OK;
    }
    const int threads = fwd_threads(rows, s, true);
    const unsigned grid = fwd_grid(rows, s, threads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* y16 = static_cast<half_t*>(y);
    auto* x16 = static_cast<const half_t*>(x);
    auto* g16 = static_cast<const half_t*>(gamma);
    auto* b16 = static_cast<const half_t*>(beta);
    fz.z = static_cast<half_t*>(z);
    fz.bias = static_cast<const half_t*>(bias);
    fz.residual = static_cast<const half_t*>(residual);
    const uint32_t r32 = static_cast<uint32_t>(rows), h32 = static_cast<uint32_t>(hidden);
    clear_hip_error();
    LS_LN_TABLE(LS_LN_FWD_FUSED)
    char buf[112];
    snprintf(buf, sizeof(buf), "bias_dropout_residual_layernorm/%s_b%d", s.name, threads);
    set_dispatch(buf);
    return launch_status(name);
}

size_t ls_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
    if (rows <= 0 || hidden <= 0 || hidden > ls::kMaxHidden) return 0;
    // A header (the partial-row count), then the partial rows: an upper bound
    // over every launch shape of (rows, hidden).
    return ls::kBwdHeaderBytes + static_cast<size_t>(ls::bwd_max_blocks(rows)) * 2 * static_cast<size_t>(hidden) *
                                     sizeof(float);
}

int ls_layernorm_bwd_input(void* dx, const void* dy, const void* x, const void* gamma, const float* mean,
                           const float* rstd, int64_t rows, int64_t hidden, void* workspace, size_t workspace_bytes,
                           void* stream) {
    using namespace ls;
    const char* name = "ls_layernorm_bwd_input";
    if (rows < 0 || hidden < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (rows == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (hidden == 0) return fail(LS_ERR_SHAPE, "%s: hidden must be >= 1", name);
    if (hidden > kMaxHidden)
        return fail(LS_ERR_UNSUPPORTED, "%s: hidden %lld > %lld", name, (long long)hidden, (long long)kMaxHidden);
    if (rows >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: rows must be < 2^31", name);   // 32-bit row loops
    if (!dx || !dy || !x || !gamma || !mean || !rstd || !workspace)
        return fail(LS_ERR_NULL, "%s: null pointer", name);
    const size_t need = ls_layernorm_bwd_workspace_bytes(rows, hidden);
    if (workspace_bytes < need)
        return fail(LS_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", name, workspace_bytes, need);
    if (!aligned16(workspace)) return fail(LS_ERR_PARAM, "%s: workspace must be 16-byte aligned", name);
    const bool vec = hidden % 8 == 0 && aligned16(dx) && aligned16(dy) && aligned16(x) && aligned16(gamma);
    LnShape s;
    ln_shape(hidden, vec, &s);
    const BwdLaunch bl = bwd_launch(rows, hidden, s);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto* dx16 = static_cast<half_t*>(dx);
    auto* dy16 = static_cast<const half_t*>(dy);
    auto* x16 = static_cast<const half_t*>(x);
    auto* g16 = static_cast<const half_t*>(gamma);
    auto* hdr = static_cast<uint32_t*>(workspace);
    auto* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kBwdHeaderBytes);
    const uint32_t r32 = static_cast<uint32_t>(rows), h32 = static_cast<uint32_t>(hidden);
    clear_hip_error();
    LS_LN_TABLE(LS_LN_BWD)
    char buf[96];
    snprintf(buf, sizeof(buf), "layernorm_bwd/%s_w%d_g%u", s.name, bl.waves, bl.grid);
    set_dispatch(buf);
    return launch_status(name);
}

int ls_layernorm_bwd_params_batched(int count, void* const* dgamma, void* const* dbeta, const int64_t* rows,
                                    const int64_t* hidden, void* const* workspace, const size_t* workspace_bytes,
                                    void* stream) {
    using namespace ls;
    const char* name = "ls_layernorm_bwd_params_batched";
    if (count < 0) return fail(LS_ERR_PARAM, "%s: negative count", name);
    if (count > 0 && (!dgamma || !dbeta || !rows || !hidden || !workspace || !workspace_bytes))
        return fail(LS_ERR_NULL, "%s: null array", name);
    // Every job is checked before anything is launched.
    for (int i = 0; i < count; ++i) {
        char who[80];
        snprintf(who, sizeof(who), "%s: job %d", name, i);
        if (const int rc = check_params_job(who, dgamma[i], dbeta[i], rows[i], hidden[i], workspace[i],
                                            workspace_bytes[i]))
            return rc;
    }
    if (launch_params_jobs(count, dgamma, dbeta, rows, hidden, workspace, static_cast<hipStream_t>(stream)) == 0)
        return LS_OK;
    return launch_status(name);
}

int ls_layernorm_bwd_params(void* dgamma, void* dbeta, int64_t rows, int64_t hidden, const void* workspace,
                            size_t workspace_bytes, void* stream) {
    using namespace ls;
    const char* name = "ls_layernorm_bwd_params";
    if (const int rc = check_params_job(name, dgamma, dbeta, rows, hidden, workspace, workspace_bytes)) return rc;
    void* ws = const_cast<void*>(workspace);
    if (launch_params_jobs(1, &dgamma, &dbeta, &rows, &hidden, &ws, static_cast<hipStream_t>(stream)) == 0)
        return LS_OK;
    const int rc = launch_status(name);
    set_dispatch(rows > 0 ? "layernorm_bwd_params/fixed_order" : "layernorm_bwd_params/zero_rows");
    return rc;
}

size_t ls_layernorm_bwd_noalloc_max_bytes(void) { return ls::kScratchBytes; }

int ls_layernorm_bwd_noalloc(void* dx, void* dgamma, void* dbeta, const void* dy, const void* x,
                             const void* gamma, const float* mean, const float* rstd, int64_t rows,
                             int64_t hidden, void* stream) {
    using namespace ls;
    const char* name = "ls_layernorm_bwd_noalloc";
    if (rows < 0 || hidden < 0) return fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (hidden > kMaxHidden)
        return fail(LS_ERR_UNSUPPORTED, "%s: hidden %lld > %lld", name, (long long)hidden, (long long)kMaxHidden);
    const size_t need = ls_layernorm_bwd_workspace_bytes(rows, hidden);
    if (need > kScratchBytes)
        return fail(LS_ERR_WORKSPACE,
                    "%s: [%lld, %lld] needs %zu bytes of scratch, more than the %zu this entry point holds "
                    "(use ls_layernorm_bwd with a workspace)",
                    name, (long long)rows, (long long)hidden, need, kScratchBytes);
    void* ws = nullptr;
    if (rows > 0 && hidden > 0) {
        if (const int rc = scratch_for_current_device(name, &ws)) return rc;
    }
    return ls_layernorm_bwd(dx, dgamma, dbeta, dy, x, gamma, mean, rstd, rows, hidden, ws, kScratchBytes,
                            stream);
}

int ls_layernorm_bwd(void* dx, void* dgamma, void* dbeta, const void* dy, const void* x,
                     const void* gamma, const float* mean, const float* rstd, int64_t rows,
                     int64_t hidden, void* workspace, size_t workspace_bytes, void* stream) {
    const char* name = "ls_layernorm_bwd";
    if (rows < 0 || hidden < 0) return ls::fail(LS_ERR_SHAPE, "%s: negative shape", name);
    if (rows > 0) {
        const int rc = ls_layernorm_bwd_input(dx, dy, x, gamma, mean, rstd, rows, hidden, workspace,
                                              workspace_bytes, stream);
        if (rc != LS_OK) return rc;
    }
    char disp[128];
    snprintf(disp, sizeof(disp), "%s", ls_last_dispatch());
    const int rc = ls_layernorm_bwd_params(dgamma, dbeta, rows, hidden, workspace, workspace_bytes, stream);
    if (rc != LS_OK) return rc;
    ls::set_dispatch(rows > 0 ? disp : "layernorm_bwd/zero_rows");
    return LS_OK;
}

}  // extern "C"
