// Bias add fused with the split of the Q/K/V projection into heads ([L10]
// technique 1, slide 12 and [LS2] sec. 2.1.1 list it among the fused
// elementwise kernels of the attention block), and its inverse for the
// backward.
//
// Forward: the projection output qkv [T = B*L, 3H] holds, per token, the Q,
// K and V rows one after another, each of them heads x d (H = heads * d).
//     out[k][b][h][l][j] = qkv[b*L + l][k*H + h*d + j] + bias[k*H + h*d + j]
// with out [3, B, heads, L, d]: every head gets its own contiguous [L, d]
// tile, the layout the attention GEMMs read.
// Backward: dqkv = the inverse permutation of dout (exact), and
// dbias = the column sum of dqkv over the tokens (fixed order).
//
// Both directions move 16-byte vectors (8 consecutive j): the head dimension
// is innermost on both sides, so the permutation never splits a vector.  The
// forward reads qkv in order (each wave 1 KiB contiguous) and writes d*2-byte
// runs per head; the backward writes dqkv in order and reads those runs.
#include "colsum.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;

// Index arithmetic of the permutation, in units of 16-byte vectors.
struct QkvShape {
    FastDiv nv3;     // vectors per token row (3H/8)
    FastDiv nvh;     // vectors per Q, K or V part (H/8)
    FastDiv nvd;     // vectors per head (d/8)
    FastDiv seq;     // L
    uint32_t batch, heads;
    // Output vector index of (part k, sequence b, head h, position l, vector j).
    __device__ __forceinline__ uint32_t out_index(uint32_t k, uint32_t b, uint32_t h, uint32_t l, uint32_t j) const {
        return (((k * batch + b) * heads + h) * seq.d + l) * nvd.d + j;
    }
};

__global__ __launch_bounds__(kBlock) void qkv_split_vec_kernel(half8* out, const half8* qkv, const half8* bias,
                                                               uint32_t nvec, QkvShape s) {
    const uint32_t v = blockIdx.x * kBlock + threadIdx.x;
    if (v >= nvec) return;
    const half8 x = __builtin_nontemporal_load(qkv + v);
    const uint32_t t = s.nv3.div(v);
    const uint32_t cv = v - t * s.nv3.d;
    const half8 bv = bias[cv];
    const uint32_t k = s.nvh.div(cv);
    const uint32_t rem = cv - k * s.nvh.d;
    const uint32_t h = s.nvd.div(rem);
    const uint32_t j = rem - h * s.nvd.d;
    const uint32_t b = s.seq.div(t);
    const uint32_t l = t - b * s.seq.d;
    float a[8], c[8];
    unpack8(x, a);
    unpack8(bv, c);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] += c[e];
    __builtin_nontemporal_store(pack8(a), out + s.out_index(k, b, h, l, j));
}

// Element-wise path (head_dim % 8 != 0 or unaligned tensors), 64-bit indices.
__global__ __launch_bounds__(kBlock) void qkv_split_scalar_kernel(half_t* out, const half_t* qkv, const half_t* bias,
                                                                  uint64_t n, uint64_t batch, uint64_t seq,
                                                                  uint64_t heads, uint64_t d) {
    const uint64_t hid = heads * d, cols = 3 * hid;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n; i += stride) {
        const uint64_t t = i / cols, c = i % cols;
        const uint64_t k = c / hid, h = (c % hid) / d, j = c % d;
        const uint64_t b = t / seq, l = t % seq;
        const float y = static_cast<float>(qkv[i]) + static_cast<float>(bias[c]);
        out[(((k * batch + b) * heads + h) * seq + l) * d + j] = to_half(y);
    }
}

// Backward, vector path: block (segment of 64 column vectors, row group);
// lane = one column vector of dqkv, i.e. a fixed (k, h, j); rows = tokens.
__global__ __launch_bounds__(kCsBlock) void qkv_split_bwd_vec_kernel(half8* dqkv, float* partial, const half8* dout,
                                                                     uint32_t tokens, uint32_t rows_per_group,
                                                                     QkvShape s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t cv = blockIdx.x * kSegVecs + lane;
    const bool col_ok = cv < s.nv3.d;
    const uint32_t k = s.nvh.div(cv);
    const uint32_t rem = cv - k * s.nvh.d;
    const uint32_t h = s.nvd.div(rem);
    const uint32_t j = rem - h * s.nvd.d;
    const uint32_t r_begin = blockIdx.y * rows_per_group;
    const uint32_t r_end = min(tokens, r_begin + rows_per_group);
    auto src = [&](uint32_t t) {
        const uint32_t b = s.seq.div(t);
        return s.out_index(k, b, h, t - b * s.seq.d, j);
    };

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    uint32_t t = r_begin + wave;
    half8 g{};
    if (col_ok && t < r_end) g = __builtin_nontemporal_load(dout + src(t));
    for (; t < r_end; t += kCsWaves) {
        const uint32_t tn = t + kCsWaves;
        half8 gn{};
        if (col_ok && tn < r_end) gn = __builtin_nontemporal_load(dout + src(tn));   // next row first
        if (col_ok) {
            float f[8];
            unpack8(g, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += f[e];
            __builtin_nontemporal_store(g, dqkv + static_cast<size_t>(t) * s.nv3.d + cv);
        }
        g = gn;
    }
    colsum_block_fold(partial, acc, s.nv3.d * 8u);
}

__global__ __launch_bounds__(256) void qkv_split_bwd_scalar_kernel(half_t* dqkv, float* partial, const half_t* dout,
                                                                   uint64_t tokens, uint64_t rows_per_group,
                                                                   uint64_t batch, uint64_t seq, uint64_t heads,
                                                                   uint64_t d) {
    const uint64_t hid = heads * d, cols = 3 * hid;
    const uint64_t c = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (c >= cols) return;
    const uint64_t k = c / hid, h = (c % hid) / d, j = c % d;
    const uint64_t r_begin = static_cast<uint64_t>(blockIdx.y) * rows_per_group;
    const uint64_t r_end = tokens < r_begin + rows_per_group ? tokens : r_begin + rows_per_group;
    float acc = 0.0f;
    for (uint64_t t = r_begin; t < r_end; ++t) {
        const uint64_t b = t / seq, l = t % seq;
        const half_t g = dout[(((k * batch + b) * heads + h) * seq + l) * d + j];
        acc += static_cast<float>(g);
        dqkv[t * cols + c] = g;
    }
    partial[static_cast<size_t>(blockIdx.y) * cols + c] = acc;
}

// Shared validation: 0 = proceed, else the (negated) status of the failure.
int qkv_check(const char* name, int64_t batch, int64_t seq, int64_t heads, int64_t d) {
    if (batch < 0 || seq < 0 || heads < 0 || d < 0) return -fail(LS_ERR_SHAPE, "%s: negative size", name);
    if (heads > (1ll << 20) || d > (1ll << 20) || batch > (1ll << 31) || seq > (1ll << 31))
        return -fail(LS_ERR_SHAPE, "%s: size too large", name);
    const int64_t cols = 3 * heads * d;
    if (cols > 0 && batch * seq > INT64_MAX / cols) return -fail(LS_ERR_SHAPE, "%s: size too large", name);
    return 0;
}

bool qkv_vec_ok(int64_t tokens, int64_t cols, int64_t d) {
    return d % 8 == 0 && static_cast<uint64_t>(tokens) * static_cast<uint64_t>(cols) / 8 < (1ull << 31);
}

QkvShape qkv_shape(int64_t batch, int64_t seq, int64_t heads, int64_t d) {
    QkvShape s;
    s.nv3 = FastDiv(static_cast<uint32_t>(3 * heads * d / 8));
    s.nvh = FastDiv(static_cast<uint32_t>(heads * d / 8));
    s.nvd = FastDiv(static_cast<uint32_t>(d / 8));
    s.seq = FastDiv(static_cast<uint32_t>(seq));
    s.batch = static_cast<uint32_t>(batch);
    s.heads = static_cast<uint32_t>(heads);
    return s;
}

}  // namespace
}  // namespace ls

extern "C" {

int ls_bias_qkv_split(void* out, const void* qkv, const void* bias, int64_t batch, int64_t seq_len, int64_t heads,
                      int64_t head_dim, void* stream) {
    using namespace ls;
    const char* name = "ls_bias_qkv_split";
    if (int rc = qkv_check(name, batch, seq_len, heads, head_dim)) return -rc;
    const int64_t tokens = batch * seq_len, cols = 3 * heads * head_dim;
    if (tokens == 0 || cols == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!out || !qkv || !bias) return fail(LS_ERR_NULL, "%s: null pointer", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    clear_hip_error();
    const uint64_t n = static_cast<uint64_t>(tokens) * static_cast<uint64_t>(cols);
    if (qkv_vec_ok(tokens, cols, head_dim) && aligned16(out) && aligned16(qkv) && aligned16(bias)) {
        const uint32_t nvec = static_cast<uint32_t>(n / 8);
        qkv_split_vec_kernel<<<(nvec + kBlock - 1) / kBlock, kBlock, 0, st>>>(
            static_cast<half8*>(out), static_cast<const half8*>(qkv), static_cast<const half8*>(bias), nvec,
            qkv_shape(batch, seq_len, heads, head_dim));
        set_dispatch("bias_qkv_split/vec8");
    } else {
        const uint64_t blocks = (n + kBlock - 1) / kBlock;
        qkv_split_scalar_kernel<<<static_cast<unsigned>(blocks < 65536 ? blocks : 65536), kBlock, 0, st>>>(
            static_cast<half_t*>(out), static_cast<const half_t*>(qkv), static_cast<const half_t*>(bias), n,
            static_cast<uint64_t>(batch), static_cast<uint64_t>(seq_len), static_cast<uint64_t>(heads),
            static_cast<uint64_t>(head_dim));
        set_dispatch("bias_qkv_split/scalar");
    }
    return launch_status(name);
}

int ls_bias_qkv_split_bwd(void* dqkv, void* dbias, const void* dout, int64_t batch, int64_t seq_len, int64_t heads,
                          int64_t head_dim, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace ls;
    const char* name = "ls_bias_qkv_split_bwd";
    if (int rc = qkv_check(name, batch, seq_len, heads, head_dim)) return -rc;
    const int64_t tokens = batch * seq_len, cols = 3 * heads * head_dim;
    if (cols == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    if (!dbias) return fail(LS_ERR_NULL, "%s: null dbias", name);
    if (cols >= (1ll << 31) || tokens >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: shape too large", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    clear_hip_error();
    if (tokens == 0) {
        colsum_finalize(static_cast<half_t*>(dbias), nullptr, 0, static_cast<uint32_t>(cols), st);
        set_dispatch("bias_qkv_split_bwd/empty_rows");
        return launch_status(name);
    }
    if (!dqkv || !dout) return fail(LS_ERR_NULL, "%s: null pointer", name);
    if (int rc = colsum_check_workspace(name, workspace, workspace_bytes, tokens, cols)) return rc;
    const uint32_t groups = colsum_groups(tokens, cols);
    const uint64_t rpg = (static_cast<uint64_t>(tokens) + groups - 1) / groups;
    float* part = static_cast<float*>(workspace);
    char buf[96];
    if (qkv_vec_ok(tokens, cols, head_dim) && aligned16(dqkv) && aligned16(dout)) {
        const uint32_t nv3 = static_cast<uint32_t>(cols / 8);
        const dim3 grid((nv3 + kSegVecs - 1) / kSegVecs, groups);
        qkv_split_bwd_vec_kernel<<<grid, kCsBlock, 0, st>>>(static_cast<half8*>(dqkv), part,
                                                            static_cast<const half8*>(dout),
                                                            static_cast<uint32_t>(tokens), static_cast<uint32_t>(rpg),
                                                            qkv_shape(batch, seq_len, heads, head_dim));
        snprintf(buf, sizeof(buf), "bias_qkv_split_bwd/seg512_w16_g%u", groups);
    } else {
        const dim3 grid(static_cast<unsigned>((cols + 255) / 256), groups);
        qkv_split_bwd_scalar_kernel<<<grid, 256, 0, st>>>(static_cast<half_t*>(dqkv), part,
                                                         static_cast<const half_t*>(dout),
                                                         static_cast<uint64_t>(tokens), rpg,
                                                         static_cast<uint64_t>(batch), static_cast<uint64_t>(seq_len),
                                                         static_cast<uint64_t>(heads), static_cast<uint64_t>(head_dim));
        snprintf(buf, sizeof(buf), "bias_qkv_split_bwd/scalar_g%u", groups);
    }
    int rc = launch_status(name);
    if (rc != LS_OK) return rc;
    colsum_finalize(static_cast<half_t*>(dbias), part, groups, static_cast<uint32_t>(cols), st);
    set_dispatch(buf);
    return launch_status(name);
}

}  // extern "C"
