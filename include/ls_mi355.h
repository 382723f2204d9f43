/*
 * ls_mi355 -- fused memory-bound non-GEMM Transformer operators for MI355X
 * (gfx950, CDNA4), hand-written HIP behind a plain C ABI.
 *
 * Sources (cited by page title and section):
 *   [L10]   CMU 11-868 L10 digest, "Accelerating Transformer on GPU: where
 *           LightSeq saves its time" (quidproquo.cc): technique 1, kernel
 *           fusion (slide 12); technique 2, formula rewriting for LayerNorm
 *           and softmax (slides 21-26); technique 3, the fp16 workspace
 *           trainer (slide 29).
 *   [LS2]   "LightSeq2: Accelerated Training for Transformer-based Models
 *           on GPUs", reading notes (arcsin2.cloud): sec. 2.1.1 (operator
 *           classes, fused bias/dropout/residual), sec. 2.1.2 (embedding
 *           forward and backward equations), sec. 2.3 (mixed-precision
 *           trainer, symbolic tensor linking).
 *   [CS336] Stanford CS336 lecture 5 notes, "GPU" (auss.cc): sec. 3.2
 *           (loss scaling).
 *   [SC11]  Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3"
 *           (Philox4x32-10).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense and row-major.  "fp16" means IEEE binary16 storage,
 *    passed as void*; all arithmetic is fp32 in registers, results are
 *    rounded to fp16 with round-to-nearest-even.  fp16 subnormals are kept.
 *  - Every tensor pointer is a DEVICE pointer into memory the caller owns.
 *    The library never allocates, frees or synchronises; it keeps no device
 *    state.  `stream` is a hipStream_t passed as void* (NULL = null stream);
 *    every call only enqueues work on it.
 *  - Each call validates its arguments on the host first and returns a
 *    non-zero ls_status without launching anything if they are invalid; the
 *    reason is available from ls_last_error() (thread-local).  A failed
 *    launch returns LS_ERR_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation, as usual for HIP.
 *  - A tensor with zero elements is a valid no-op (its pointers may then be
 *    NULL).  Negative sizes are LS_ERR_SHAPE.
 *  - Unaligned pointers (not 16-byte aligned) or a last dimension that is not
 *    a multiple of 8 select a slower element-wise path; they are not errors.
 *  - Aliasing: the pairs named in each comment may be the same buffer; any
 *    other overlap is undefined.
 *  - Calls are re-entrant and thread-safe.
 *
 * Dropout
 * -------
 *  Dropout is inverted (kept values are scaled by 1/(1-p_eff) at training
 *  time) and counter based: element i of a dropout site is decided by a
 *  16-bit field of Philox4x32-10 [SC11] with key (lo32(seed), hi32(seed))
 *  and counter (lo32(i/8), hi32(i/8), lo32(offset), hi32(offset)); field
 *  i%8 is taken from output word (i%8)/2, low half first.  The element is
 *  dropped iff field < floor(p * 65536), so p_eff = floor(p*65536)/65536
 *  (|p - p_eff| < 2^-16).  `offset` separates dropout sites that share a
 *  seed.  The same (seed, offset) regenerates the same mask in a backward
 *  pass, so no mask is stored.  i is the flat row-major index of the
 *  operator's output element.  p must lie in [0, 1]; p = 1 drops everything.
 */
#ifndef LS_MI355_H
#define LS_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LS_OK = 0,
    LS_ERR_NULL = 1,          /* a required pointer is NULL                  */
    LS_ERR_SHAPE = 2,         /* a size is negative, zero where not allowed,
                                 or too large for the index arithmetic       */
    LS_ERR_PARAM = 3,         /* a scalar argument is out of its domain      */
    LS_ERR_WORKSPACE = 4,     /* caller-provided workspace is too small      */
    LS_ERR_UNSUPPORTED = 5,   /* shape outside what the kernels implement    */
    LS_ERR_HIP = 6,           /* the HIP runtime reported an error           */
    LS_ERR_UNIMPLEMENTED = 7
} ls_status;

/* Fused bias + dropout + residual ([L10] technique 1; [LS2] sec. 2.1.1, the
 * fused tail of the self-attention block):
 *     out[r,c] = residual[r,c] + keep(r*cols+c) * (x[r,c] + bias[c]) / (1-p_eff)
 * x, residual, out: fp16 [rows, cols]; bias: fp16 [cols].
 * out may alias x or residual.  p in [0, 1]. */
int ls_bias_dropout_residual(void* out, const void* x, const void* bias, const void* residual,
                             int64_t rows, int64_t cols, float p, uint64_t seed, uint64_t offset,
                             void* stream);

/* Fused bias + ReLU + dropout ([L10] technique 1, slide 12):
 *     out[r,c] = keep(r*cols+c) * max(x[r,c] + bias[c], 0) / (1-p_eff)
 * x, out: fp16 [rows, cols]; bias: fp16 [cols].  out may alias x. */
int ls_bias_relu_dropout(void* out, const void* x, const void* bias, int64_t rows, int64_t cols,
                         float p, uint64_t seed, uint64_t offset, void* stream);

/* Backward of the two operators above (their derivatives; [L10] technique 1
 * and [LS2] sec. 2.1.1 fuse each operator in both directions).
 *
 * ls_bias_dropout_residual_bwd:
 *     dx[r,c]   = dy[r,c] * keep(r*cols+c) / (1-p_eff)   (gradient of x and
 *                 of the branch x + bias; the mask is regenerated from the
 *                 forward's seed and offset)
 *     dbias[c]  = sum_r dx[r,c]    (of the fp32 values, before rounding dx)
 *     d_residual = dy: nothing is computed for it.
 * ls_bias_relu_dropout_bwd:
 *     dx[r,c]   = dy[r,c] * [out[r,c] > 0] / (1-p_eff),  dbias[c] = sum_r dx[r,c]
 *   where out is the forward's output: for fp16 inputs out > 0 exactly when
 *   the element was kept and x + bias > 0, so no random numbers are drawn;
 *   p must be the forward's.
 * dy, dx, out: fp16 [rows, cols]; dbias: fp16 [cols].  dx may alias dy (or
 * out).  dbias is reduced in a fixed order (bit-reproducible).  rows == 0
 * writes zeros to dbias; cols == 0 is a no-op.
 * workspace: device memory of at least
 * ls_elementwise_bwd_workspace_bytes(rows, cols) bytes (fp32 partial column
 * sums), 16-byte aligned, not shared with a call that may run concurrently;
 * its contents need no initialisation.  Errors: LS_ERR_WORKSPACE if too
 * small; LS_ERR_PARAM for p outside [0, 1] or a misaligned workspace;
 * LS_ERR_SHAPE for rows or cols >= 2^31. */
size_t ls_elementwise_bwd_workspace_bytes(int64_t rows, int64_t cols);
int ls_bias_dropout_residual_bwd(void* dx, void* dbias, const void* dy, int64_t rows, int64_t cols,
                                 float p, uint64_t seed, uint64_t offset, void* workspace,
                                 size_t workspace_bytes, void* stream);
int ls_bias_relu_dropout_bwd(void* dx, void* dbias, const void* dy, const void* out, int64_t rows,
                             int64_t cols, float p, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Bias add fused with the split of the Q/K/V projection into heads, and its
 * inverse for the backward ([L10] technique 1, slide 12; [LS2] sec. 2.1.1
 * lists it with the fused elementwise kernels of the attention block).
 * T = batch * seq_len tokens, H = heads * head_dim.
 *
 * ls_bias_qkv_split:
 *     out[k][b][h][l][j] = qkv[b*seq_len + l][k*H + h*head_dim + j]
 *                          + bias[k*H + h*head_dim + j]
 *   qkv: fp16 [T, 3H], each token row holding its Q, K and V parts in that
 *   order, each part heads x head_dim; bias: fp16 [3H];
 *   out: fp16 [3, batch, heads, seq_len, head_dim] (Q, K, V, one contiguous
 *   [seq_len, head_dim] tile per head).  No aliasing.
 * ls_bias_qkv_split_bwd:
 *     dqkv[b*seq_len + l][k*H + h*head_dim + j] = dout[k][b][h][l][j]
 *     dbias[c] = sum over tokens of dqkv[t][c]   (fp32, fixed order)
 *   dout: fp16 [3, batch, heads, seq_len, head_dim]; dqkv: fp16 [T, 3H]
 *   (an exact permutation of dout); dbias: fp16 [3H].  No aliasing.
 *   workspace: at least ls_elementwise_bwd_workspace_bytes(T, 3H) bytes,
 *   16-byte aligned, not shared with a concurrent call; no initialisation.
 *   T == 0 writes zeros to dbias; H == 0 is a no-op.
 * head_dim % 8 == 0 with 16-byte aligned pointers takes the vector path.
 * Errors: LS_ERR_SHAPE for negative or too large sizes, LS_ERR_NULL,
 * LS_ERR_WORKSPACE, LS_ERR_PARAM for a misaligned workspace. */
int ls_bias_qkv_split(void* out, const void* qkv, const void* bias, int64_t batch, int64_t seq_len,
                      int64_t heads, int64_t head_dim, void* stream);
int ls_bias_qkv_split_bwd(void* dqkv, void* dbias, const void* dout, int64_t batch, int64_t seq_len,
                          int64_t heads, int64_t head_dim, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Cross-entropy criterion with label smoothing over vocabulary rows ([L10]
 * technique 1, slide 12 lists it among the fused reduce kernels; [LS2]
 * sec. 2.1.3 defers its details to the slides).  Per row t of logits x
 * (fp16 [rows, vocab]) with target y_t (int32 [rows]) and smoothing eps:
 *     lse[t]  = log sum_j exp(x[t,j])                               (fp32)
 *     loss[t] = lse[t] - (1-eps)*x[t,y_t] - eps*mean_j x[t,j]       (fp32)
 *     dlogits[t,j] = grad_scale * (exp(x[t,j] - lse[t])
 *                                  - (1-eps)*[j == y_t] - eps/vocab) (fp16)
 * eps = 0 is the plain negative log-likelihood.  A row whose target equals
 * ignore_index has loss 0 and a zero gradient; any other target outside
 * [0, vocab) gives a NaN loss and NaN gradients for its row.  NaN or +inf
 * logits give NaN.  The forward reads each row once (one-pass running max
 * and sum, [CS336] sec. 6.2), reduces in a fixed order, and saves lse for
 * the backward, which takes the forward's lse.  dlogits may alias logits.
 * eps in [0, 1]; grad_scale finite; rows, vocab < 2^31.
 * Errors: LS_ERR_SHAPE, LS_ERR_PARAM, LS_ERR_NULL. */
int ls_cross_entropy_fwd(float* loss, float* lse, const void* logits, const int32_t* targets,
                         int64_t rows, int64_t vocab, float smoothing, int32_t ignore_index,
                         void* stream);
int ls_cross_entropy_bwd(void* dlogits, const void* logits, const int32_t* targets, const float* lse,
                         int64_t rows, int64_t vocab, float smoothing, int32_t ignore_index,
                         float grad_scale, void* stream);

/* Beam-search top-k by hierarchical filtering (HARS, the inference part of
 * [L10], beam search slides 45-54).  For each batch element b the
 * candidates are
 *     c[i, v] = log_probs[b, i, v] + beam_scores[b, i]     (one fp32 add)
 * over beams i < beam and vocabulary entries v < vocab; the call returns
 * the k largest, in descending order, ties broken by the smaller flat index
 * i * vocab + v: top_scores fp32 [batch, k] and top_ids int32 [batch, k]
 * (flat indices).  Ordering is total: every NaN ranks above +inf and -0
 * below +0; a NaN score is returned as the default quiet NaN.  beam_scores
 * may be NULL: then c = log_probs exactly.
 * Steps, per beam: its candidates split into k groups, the smallest group
 * maximum bounds the beam's k-th best from below, only candidates at or
 * above it are kept and sorted, and the beam's best k go to the workspace;
 * then the beam x k winners of each batch element are sorted.  Heavily tied
 * rows (more than 4096 survivors) fall back to k exact selection passes,
 * with the same result.
 * log_probs: fp32 [batch, beam, vocab].  1 <= k <= min(1024, beam*vocab),
 * beam * k <= 4096, beam * vocab < 2^31.  workspace: device memory of
 * ls_beam_topk_workspace_bytes(batch, beam, k) bytes, 8-byte aligned, no
 * initialisation, not shared with a concurrent call.
 * Errors: LS_ERR_SHAPE, LS_ERR_UNSUPPORTED (k > 1024 or beam * k > 4096),
 * LS_ERR_NULL, LS_ERR_WORKSPACE, LS_ERR_PARAM (misaligned workspace). */
size_t ls_beam_topk_workspace_bytes(int64_t batch, int64_t beam, int64_t k);
int ls_beam_topk(float* top_scores, int32_t* top_ids, const float* log_probs, const float* beam_scores,
                 int64_t batch, int64_t beam, int64_t vocab, int64_t k, void* workspace,
                 size_t workspace_bytes, void* stream);

/* LayerNorm forward with one fused reduction pass ([L10] technique 2,
 * slide 21): per row, with d = x - K and K the row's first element,
 * S1 = sum d and S2 = sum d^2 are reduced together; mean = K + S1/H,
 * var = max(S2/H - (S1/H)^2, 0), rstd = 1/sqrt(var + eps),
 * y = (x - mean) * rstd * gamma + beta.  (The shift K leaves the one-pass
 * formula exact in real arithmetic and keeps the fp32 statistics accurate
 * on rows whose |mean| is large next to their spread.)
 * x, y: fp16 [rows, hidden]; gamma, beta: fp16 [hidden];
 * mean, rstd: fp32 [rows] (saved for the backward).  y may alias x.
 * eps > 0.  hidden must be in [1, 4096]; rows < 2^31 (else LS_ERR_SHAPE).
 * rows == 0 launches nothing. */
int ls_layernorm_fwd(void* y, float* mean, float* rstd, const void* x, const void* gamma,
                     const void* beta, int64_t rows, int64_t hidden, float eps, void* stream);

/* Bias + dropout + residual followed by LayerNorm, in one launch: the
 * sub-layer output block of a post-LN Transformer layer ([LS2] sec. 2.1.1;
 * [L10] technique 1 fuses neighbouring memory-bound operators).
 *     z = residual + Dropout(x + bias)      (exactly ls_bias_dropout_residual)
 *     (y, mean, rstd) = LayerNorm(z)        (exactly ls_layernorm_fwd of z)
 * z is rounded to fp16 and stored (the LayerNorm backward reads it), and the
 * statistics are those of the stored z; z is not read back from memory.  z
 * is bit-identical to ls_bias_dropout_residual's output; y, mean and rstd
 * equal ls_layernorm_fwd's of that z up to the order of the fp32 sums (rows
 * of 65-96 16-byte vectors take 32 lanes each here, 64 there).
 * x, residual, z, y: fp16 [rows, hidden]; bias, gamma, beta: fp16 [hidden];
 * mean, rstd: fp32 [rows].  Dropout as in ls_bias_dropout_residual (flat
 * element index row * hidden + col, site `offset`).  z may alias x or
 * residual; y must not alias any input.
 * p in [0, 1], eps > 0, hidden in [1, 4096], rows < 2^31.
 * One launch; element-wise rows (hidden % 8 != 0 or a pointer not 16-byte
 * aligned) longer than 2048 take the two standalone operators' launches.
 * Errors: LS_ERR_SHAPE, LS_ERR_PARAM, LS_ERR_UNSUPPORTED (hidden > 4096),
 * LS_ERR_NULL.  rows == 0 launches nothing. */
int ls_bias_dropout_residual_layernorm(void* z, void* y, float* mean, float* rstd, const void* x,
                                       const void* bias, const void* residual, const void* gamma,
                                       const void* beta, int64_t rows, int64_t hidden, float p, uint64_t seed,
                                       uint64_t offset, float eps, void* stream);

/* Bytes of device scratch that ls_layernorm_bwd needs for this shape: a
 * 256-byte header (the partial-row count) and the per-block fp32 column
 * partials of dgamma and dbeta.  Depends only on (rows, hidden).  Returns 0
 * for invalid or empty shapes. */
size_t ls_layernorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);

/* LayerNorm backward ([L10] technique 2, slide 22).  With
 * xhat = (x - mean) * rstd and g = gamma * dy, the two row sums
 * A = sum g and B = sum g * xhat are reduced together, then
 *     dx = rstd * (g - A/H - xhat * B/H).
 * dgamma = sum_rows dy * xhat and dbeta = sum_rows dy are reduced over rows
 * in a fixed order (bit-reproducible run to run).
 * dy, x, dx: fp16 [rows, hidden]; gamma: fp16 [hidden]; dgamma, dbeta: fp16
 * [hidden]; mean, rstd: fp32 [rows] from ls_layernorm_fwd.  dx may alias dy.
 * workspace: device scratch of at least ls_layernorm_bwd_workspace_bytes()
 * bytes, 16-byte aligned; its contents on entry are ignored.
 * rows < 2^31 (else LS_ERR_SHAPE).  rows == 0 writes zeros to dgamma and
 * dbeta (the sum over no rows; workspace may then be NULL) and touches
 * nothing else.
 * Exactly ls_layernorm_bwd_input followed by ls_layernorm_bwd_params on the
 * same stream: two kernel launches (row pass, then column finalisation). */
int ls_layernorm_bwd(void* dx, void* dgamma, void* dbeta, const void* dy, const void* x,
                     const void* gamma, const float* mean, const float* rstd, int64_t rows,
                     int64_t hidden, void* workspace, size_t workspace_bytes, void* stream);

/* ls_layernorm_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the header and partial rows live in a
 * file-scope device array of ls_layernorm_bwd_noalloc_max_bytes() bytes
 * (256 + 2 MiB), one copy per GPU, held until the process ends.  The call
 * allocates and frees nothing.  Shapes whose ls_layernorm_bwd_workspace_bytes
 * exceed that size (hidden > 1024 with more than 2^18 / hidden rows) return
 * LS_ERR_WORKSPACE before launching.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, different
 * host threads) race and give undefined results; calls ordered on one
 * stream are safe (nothing in the array needs clearing between calls: each
 * call writes what it later reads).  Otherwise exactly ls_layernorm_bwd:
 * same arguments minus the workspace, same results, same errors. */
size_t ls_layernorm_bwd_noalloc_max_bytes(void);
int ls_layernorm_bwd_noalloc(void* dx, void* dgamma, void* dbeta, const void* dy, const void* x,
                             const void* gamma, const float* mean, const float* rstd, int64_t rows,
                             int64_t hidden, void* stream);

/* The two halves of ls_layernorm_bwd, for callers that keep the parameter
 * gradients off the critical path: only the input gradient dx feeds the
 * rest of the backward pass, while dgamma / dbeta wait for the optimizer, so
 * the finalisation may run on another stream (ordered after the input call
 * by an event) while the next operators proceed, or later, together with
 * other LayerNorms' (ls_layernorm_bwd_params_batched).
 * ls_layernorm_bwd_input: dx, and the fixed-order per-block column partials
 * plus their count into workspace (arguments and errors as ls_layernorm_bwd;
 * rows == 0 launches nothing).
 * ls_layernorm_bwd_params: dgamma, dbeta from the partials of the input call
 * with the same (rows, hidden) and workspace, which must be complete (same
 * stream, or an event) and not overwritten before this call runs.  rows == 0
 * writes zeros without reading the workspace (it may be NULL).  A workspace
 * not written by a matching input call gives unspecified values, but every
 * read stays inside workspace_bytes.
 * Errors: LS_ERR_SHAPE, LS_ERR_UNSUPPORTED (hidden > 4096), LS_ERR_NULL,
 * LS_ERR_WORKSPACE, LS_ERR_PARAM (misaligned workspace). */
int ls_layernorm_bwd_input(void* dx, const void* dy, const void* x, const void* gamma, const float* mean,
                           const float* rstd, int64_t rows, int64_t hidden, void* workspace, size_t workspace_bytes,
                           void* stream);
int ls_layernorm_bwd_params(void* dgamma, void* dbeta, int64_t rows, int64_t hidden, const void* workspace,
                            size_t workspace_bytes, void* stream);

/* Parameter-gradient finalisation of several LayerNorms in one launch: job i
 * is exactly ls_layernorm_bwd_params(dgamma[i], dbeta[i], rows[i], hidden[i],
 * workspace[i], workspace_bytes[i]).  A layer's (or a model's) LayerNorm
 * gradients dgamma / dbeta are read only by the optimizer ([LS2] §2.3: the
 * trainer updates the whole gradient workspace at once), so their
 * finalisations can wait and share one launch; each job's workspace must
 * hold its own input call's partials, complete and not overwritten.
 * The arrays are host arrays of `count` entries; up to 16 jobs share a
 * launch (more take several).  Jobs with hidden == 0 are skipped; rows == 0
 * writes zeros without reading that job's workspace.  The jobs' outputs must
 * not overlap one another (nor any workspace).  Every job is checked
 * before anything is launched; the first failing job's error is returned
 * (the message names the job) and nothing runs.  count == 0 launches nothing.
 * Errors: LS_ERR_PARAM (count < 0, misaligned workspace), LS_ERR_NULL (a null
 * array or pointer), and each job's errors as ls_layernorm_bwd_params. */
int ls_layernorm_bwd_params_batched(int count, void* const* dgamma, void* const* dbeta, const int64_t* rows,
                                    const int64_t* hidden, void* const* workspace, const size_t* workspace_bytes,
                                    void* stream);

/* Masked row softmax forward ([L10] slides 23-26) over attention scores
 * x, y: fp16 [batch, heads, q_len, k_len].  For row (b, h, i) the valid keys
 * are j < key_lengths[b] (clamped to [0, k_len]; all keys if key_lengths is
 * NULL) and, if causal != 0, j <= i.  y = exp(x - max) / sum(exp(x - max))
 * over valid keys, exactly 0 elsewhere; a row with no valid key is all 0.
 * key_lengths: device int32 [batch] or NULL.  y may alias x.
 * Rows longer than one wavefront's registers use a multi-wave path; k_len
 * must be at most 65536 (at most 1024 when it is not a multiple of 8). */
int ls_softmax_fwd(void* y, const void* x, int64_t batch, int64_t heads, int64_t q_len,
                   int64_t k_len, const int32_t* key_lengths, int causal, void* stream);

/* Softmax backward from the stored output: dx = y * (dy - sum_j y_j dy_j)
 * per row.  y, dy, dx: fp16 [rows, k_len].  dx may alias dy.  Same k_len
 * limits as the forward; rows < 2^31 (else LS_ERR_SHAPE). */
int ls_softmax_bwd(void* dx, const void* y, const void* dy, int64_t rows, int64_t k_len,
                   void* stream);

/* Embedding forward ([LS2] sec. 2.1.2): for token t = b*seq_len + l,
 *     out[t, c] = keep(t*hidden + c) * (scale * tok_emb[ids[t], c] + pos_emb[l, c]) / (1-p_eff)
 * ids: device int32 [batch, seq_len]; tok_emb: fp16 [vocab, hidden];
 * pos_emb: fp16 [max_pos, hidden] with max_pos >= seq_len;
 * out: fp16 [batch*seq_len, hidden].  A token id outside [0, vocab) reads
 * nothing and yields a row of NaN. */
int ls_embedding_fwd(void* out, const int32_t* ids, const void* tok_emb, const void* pos_emb,
                     int64_t batch, int64_t seq_len, int64_t hidden, int64_t vocab,
                     int64_t max_pos, float scale, float p, uint64_t seed, uint64_t offset,
                     void* stream);

/* Embedding backward ([LS2] sec. 2.1.2): for every token t with id w,
 *     grad_tok_emb[w, c] += scale * keep(t*hidden + c) / (1-p_eff) * dy[t, c]
 * Repeated ids collide on one row of the table; the collisions are summed
 * with fp32 atomic adds, after the repeats inside each chunk of tokens have
 * been added up in registers: each block sorts the (id, position) keys of a
 * 1024-token chunk (64-token chunks, sorted by one wave, when vocab >= 2^22).
 * The atomics' order is not fixed, so two runs agree to fp32 rounding, not
 * bit for bit.
 * grad_tok_emb: fp32 [vocab, hidden]; if zero_first != 0 it is zeroed first
 * (by a fill kernel on the same stream), otherwise the call accumulates.
 * dy: fp16 [batch*seq_len, hidden].  (seed, offset, p) must be those of the
 * forward.  Ids outside [0, vocab) contribute nothing.  One kernel launch
 * (two with zero_first). */
int ls_embedding_bwd(float* grad_tok_emb, const int32_t* ids, const void* dy, int64_t batch,
                     int64_t seq_len, int64_t hidden, int64_t vocab, float scale, float p,
                     uint64_t seed, uint64_t offset, int zero_first, void* stream);

/* One Adam step over one contiguous fp16 parameter/gradient workspace in a
 * single kernel launch ([L10] technique 3, slide 29; [LS2] sec. 2.3): fp16
 * parameters and gradients are widened to fp32 in registers, updated, and
 * the parameter is rounded back to fp16; no fp32 master copy exists.  With
 * t = step (>= 1) and g = grad / grad_scale ([CS336] sec. 3.2):
 *     (decoupled_wd == 0: g += weight_decay * p)
 *     m = beta1 m + (1-beta1) g ;  v = beta2 v + (1-beta2) g^2
 *     u = (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
 *     (decoupled_wd != 0: u += weight_decay * p)     -- AdamW
 *     p = p - lr * u
 * param, grad: fp16 [n]; exp_avg, exp_avg_sq: fp32 [n].
 * Constraints: lr >= 0, 0 <= beta1, beta2 < 1, eps > 0, weight_decay >= 0,
 * grad_scale > 0, step >= 1. */
int ls_adam_workspace_step(void* param, const void* grad, float* exp_avg, float* exp_avg_sq,
                           int64_t n, float lr, float beta1, float beta2, float eps,
                           float weight_decay, int64_t step, float grad_scale, int decoupled_wd,
                           void* stream);

/* --- test and introspection ------------------------------------------- */

/* keep[i] = 1 if element i is kept, 0 if dropped, for i in [0, n), using
 * exactly the decision every dropout kernel above makes.  keep: device
 * uint8 [n]. */
int ls_dropout_mask(uint8_t* keep, int64_t n, float p, uint64_t seed, uint64_t offset,
                    void* stream);

/* ---------------------------------------------------------------------
 * Bandwidth reference kernels (measurement)
 * ---------------------------------------------------------------------
 * The roofline that bounds every operator above is HBM bandwidth ([CS336]
 * sec. 2.2).  These two kernels give the bandwidth this device actually
 * reaches with the operators' access pattern (one 16-byte non-temporal
 * access per lane, one 256-thread block per 4 KiB), so that a kernel's
 * achieved GB/s can be read against it as well as against the data-sheet
 * peak.  They compute nothing the operators need.
 *
 * ls_probe_copy: dst[0, bytes) = src[0, bytes).  bytes is a multiple of 16,
 *   both pointers are 16-byte aligned device pointers, no overlap.
 * ls_probe_read: reads src[0, bytes) as fp32 and writes, for every 1 KiB of
 *   it, the sum of that KiB's 256 floats to sink (ceil(bytes / 1024) floats,
 *   16-byte aligned): 0.4 % extra traffic that keeps every load live.
 * Errors: LS_ERR_SHAPE for a negative or non-multiple-of-16 size,
 *   LS_ERR_NULL for a null pointer with bytes > 0, LS_ERR_PARAM for a
 *   pointer that is not 16-byte aligned.  bytes == 0 is a no-op. */
int ls_probe_copy(void* dst, const void* src, int64_t bytes, void* stream);
int ls_probe_read(float* sink, const void* src, int64_t bytes, void* stream);

/* Kernel timing hook.  Arms two HIP events (hipEvent_t passed as void*) for
 * the calling thread's next operator call: if that call's first kernel is
 * launched through the hook (ls_bias_dropout_residual, ls_bias_relu_dropout,
 * ls_layernorm_fwd, ls_bias_dropout_residual_layernorm, ls_layernorm_bwd and
 * ls_layernorm_bwd_input: their row kernel), the launch goes through
 * hipExtLaunchKernel, which records start_event when the kernel begins and
 * stop_event when it ends, on the call's stream.  hipEventElapsedTime(start,
 * stop) is then the kernel's own duration, without the command processor's
 * handling of separate event records.  Whatever that next call does -- a
 * timed launch, another launch, no launch, or an error -- the events are
 * disarmed when it returns, so they can never attach to a later, unrelated
 * kernel.  The library neither creates, waits on nor destroys the events.
 * A NULL event disarms and returns LS_ERR_NULL. */
int ls_time_next_launch(void* start_event, void* stop_event);

/* 1 while a pair of timing events is armed for the calling thread, else 0
 * (introspection for tests). */
int ls_time_armed(void);

/* Width in bits of the random field behind one dropout decision (16). */
int ls_dropout_decision_bits(void);

/* Static text for a status code. */
const char* ls_status_string(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* ls_last_error(void);

/* Thread-local name of the kernel specialisation the last successful call on
 * this thread launched (e.g. "layernorm_fwd/lpr64_nch2_v8_b1024": 64 lanes
 * per row, 2 chunks of 8 fp16 per lane, 1024-thread blocks). */
const char* ls_last_dispatch(void);

/* Library version string. */
const char* ls_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LS_MI355_H */
