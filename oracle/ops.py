"""Plain float64 definitions of the fused non-GEMM operators.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obviously
correct: no blocking, no fusion, no one-pass rewrites.  Each function widens its
fp16 / int32 inputs to float64, computes the textbook definition, and rounds
once where the GPU path stores a value.

Readings of points the pages leave open are stated in the docstrings; they are
the same readings the library documents in its header.
"""

import numpy as np

from .philox import random_fields

# ----------------------------------------------------------------------------
# Dropout decision
# ----------------------------------------------------------------------------


def _check_p(p):
    p32 = float(np.float32(p))
    if not (0.0 <= p32 <= 1.0):
        raise ValueError("dropout probability must lie in [0, 1]")
    return p32


def drop_threshold(p, bits):
    """Integer drop threshold floor(p * 2**bits) for a bits-wide random field.

    p is taken as the float32 value the caller passes; p * 2**bits is exact in
    float64, so the floor is exact.
    """
    return int(np.floor(_check_p(p) * float(1 << bits)))


def dropout_scale(p, bits):
    """Inverted-dropout scale 1 / (1 - p_eff), p_eff = threshold / 2**bits.

    When every element is dropped (p_eff == 1) the scale is 0 so that the
    output is exactly zero.
    """
    t = drop_threshold(p, bits)
    if t >= (1 << bits):
        return 0.0
    return 1.0 / (1.0 - t / float(1 << bits))


def dropout_keep(index, p, seed, offset, bits):
    """Keep decision for each flat element index.

    Dropout is counter based: element i of one dropout site is decided by its
    own random field of the Philox4x32-10 stream keyed on ``seed`` with the
    stream word ``offset`` (one offset per dropout site), so forward and
    backward regenerate the same mask without storing it.  An element is
    dropped iff its field is below floor(p * 2**bits).  The mask m of [LS2]
    sec. 2.1.2 (embedding backward) is this decision times the inverted
    scale.

    index: 1-D integer array, or an int n meaning range(n).
    Returns a bool array (True = keep).
    """
    if np.isscalar(index):
        index = np.arange(int(index), dtype=np.uint64)
    t = drop_threshold(p, bits)
    if t == 0:
        return np.ones(np.asarray(index).shape, dtype=bool)
    fields = random_fields(index, bits, seed, offset)
    return fields >= np.uint64(t)


def _masked_scale(shape, p, seed, offset, bits):
    """keep * scale for a row-major tensor of this shape, as float64."""
    n = int(np.prod(shape))
    keep = dropout_keep(n, p, seed, offset, bits)
    return (keep.astype(np.float64) * dropout_scale(p, bits)).reshape(shape)


# ----------------------------------------------------------------------------
# Fused elementwise operators ([L10] technique 1, slide 12; [LS2] sec. 2.1.1)
# ----------------------------------------------------------------------------


def bias_dropout_residual(x, bias, residual, p, seed, offset, bits):
    """out = residual + Dropout(x + bias), rounded once to fp16.

    x, residual: fp16 [rows, cols]; bias: fp16 [cols] (broadcast over rows).
    The element index of the dropout decision is the flat row-major index.
    The order (bias add, then dropout, then residual add) is the one the
    self-attention output block of [LS2] sec. 2.1.1 fuses.
    Parity: pinned by tests (p = 0 exact sum; mask exposure with x=1, b=0, r=0;
    keep-rate statistics).
    """
    x64 = np.asarray(x, dtype=np.float64)
    b64 = np.asarray(bias, dtype=np.float64)
    r64 = np.asarray(residual, dtype=np.float64)
    ms = _masked_scale(x64.shape, p, seed, offset, bits)
    return (r64 + ms * (x64 + b64[None, :])).astype(np.float16)


def bias_relu_dropout(x, bias, p, seed, offset, bits):
    """out = Dropout(ReLU(x + bias)), rounded once to fp16 ([L10] slide 12).

    x: fp16 [rows, cols]; bias: fp16 [cols].
    Parity: pinned by tests (p = 0 equals np.maximum; zero where dropped or
    where x + b <= 0).
    """
    x64 = np.asarray(x, dtype=np.float64)
    b64 = np.asarray(bias, dtype=np.float64)
    ms = _masked_scale(x64.shape, p, seed, offset, bits)
    return (ms * np.maximum(x64 + b64[None, :], 0.0)).astype(np.float16)


def bias_dropout_residual_bwd(dy, p, seed, offset, bits):
    """Gradients of out = residual + Dropout(x + bias) (the derivative of the
    forward above; [L10] technique 1 and [LS2] sec. 2.1.1 fuse the operator in
    both directions).

    d_x = dy * keep * scale (also the gradient of the branch x + bias);
    d_bias = the column sum of d_x over rows; d_residual = dy (not returned).
    The mask is the forward's: same seed, offset and flat element index.
    d_bias sums the unrounded float64 d_x; both are rounded once to fp16.
    Returns (d_x fp16 [rows, cols], d_bias fp16 [cols]).
    Parity: pinned by tests (torch autograd of the forward in float64; p = 0
    gives d_x = dy; p = 1 gives zeros).
    """
    dy64 = np.asarray(dy, dtype=np.float64)
    dx64 = dy64 * _masked_scale(dy64.shape, p, seed, offset, bits)
    return dx64.astype(np.float16), dx64.sum(axis=0).astype(np.float16)


def bias_relu_dropout_bwd(dy, x, bias, p, seed, offset, bits):
    """Gradients of out = Dropout(ReLU(x + bias)) ([L10] slide 12's operator).

    d_x = dy * keep * scale * [x + bias > 0] (ReLU's derivative taken as 0 at
    0); d_bias = the column sum of d_x over rows.  Written from the forward's
    inputs and mask; it needs no stored output.
    Returns (d_x fp16 [rows, cols], d_bias fp16 [cols]).
    Parity: pinned by tests (torch autograd of the forward in float64; the
    gate equals [forward output > 0] for fp16 inputs; p = 0 is the plain ReLU
    gradient).
    """
    dy64 = np.asarray(dy, dtype=np.float64)
    pre = np.asarray(x, dtype=np.float64) + np.asarray(bias, dtype=np.float64)[None, :]
    dx64 = dy64 * _masked_scale(dy64.shape, p, seed, offset, bits) * (pre > 0.0)
    return dx64.astype(np.float16), dx64.sum(axis=0).astype(np.float16)


# ----------------------------------------------------------------------------
# Bias add + Q/K/V head split ([L10] technique 1, slide 12; [LS2] sec. 2.1.1)
# ----------------------------------------------------------------------------


def bias_qkv_split(qkv, bias, batch, seq_len, heads):
    """out[k, b, h, l, j] = qkv[b*L + l, k*H + h*d + j] + bias[k*H + h*d + j].

    qkv: fp16 [T, 3H] with T = batch * seq_len, each token row holding its Q,
    K and V parts in that order, each part heads x d (the layout of one
    fused [H, 3H] projection); bias: fp16 [3H].  Returns fp16
    [3, batch, heads, seq_len, d]: one contiguous [seq_len, d] tile per
    head.  The sum is rounded once to fp16.
    Parity: pinned by tests (brute-force index loops; zero bias is an exact
    permutation undone by the backward).
    """
    x = np.asarray(qkv, dtype=np.float64) + np.asarray(bias, dtype=np.float64)[None, :]
    tokens, cols = x.shape
    d = cols // (3 * heads)
    y = x.reshape(batch, seq_len, 3, heads, d).transpose(2, 0, 3, 1, 4)
    return np.ascontiguousarray(y).astype(np.float16)


def bias_qkv_split_bwd(dout, batch, seq_len, heads):
    """Gradients of bias_qkv_split: dqkv [T, 3H] is dout put back in the
    projection's layout (the inverse permutation, exact) and dbias [3H] is
    the column sum of dqkv over tokens, rounded once to fp16.
    Parity: pinned by tests (torch autograd of the forward; brute force).
    """
    g = np.asarray(dout, dtype=np.float64)
    three, b, h, l, d = g.shape
    dq = np.ascontiguousarray(g.transpose(1, 3, 0, 2, 4)).reshape(b * l, 3 * h * d)
    return dq.astype(np.float16), dq.sum(axis=0).astype(np.float16)


# ----------------------------------------------------------------------------
# Cross-entropy criterion ([L10] technique 1, slide 12; [LS2] sec. 2.1.3)
# ----------------------------------------------------------------------------


def _xent_rows(logits, targets, smoothing, ignore_index):
    x = np.asarray(logits, dtype=np.float64)
    y = np.asarray(targets, dtype=np.int64).reshape(-1)
    eps = float(np.float32(smoothing))
    if not 0.0 <= eps <= 1.0:
        raise ValueError("smoothing must lie in [0, 1]")
    m = x.max(axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))       # two passes: max, then sum
    ignored = y == ignore_index
    bad = ~ignored & ((y < 0) | (y >= x.shape[1]))
    return x, y, eps, lse, ignored, bad


def cross_entropy_fwd(logits, targets, smoothing, ignore_index):
    """Label-smoothed cross entropy per row.

    lse = log sum_j exp(x_j); loss = lse - (1 - eps) x_y - eps mean_j x_j,
    i.e. (1 - eps) (-log p_y) + eps mean_j (-log p_j).  The pages name the
    criterion and defer its details; label smoothing eps is a parameter
    (eps = 0: plain cross entropy).  A row whose target equals ignore_index
    has loss 0; any other target outside [0, V) gives NaN.
    logits fp16 [rows, V]; targets int [rows].
    Returns (loss fp32 [rows], lse fp32 [rows]).
    Parity: pinned by tests (torch.nn.functional.cross_entropy with
    label_smoothing and ignore_index in float64; scipy logsumexp).
    """
    x, y, eps, lse, ignored, bad = _xent_rows(logits, targets, smoothing, ignore_index)
    loss = np.zeros(x.shape[0])
    ok = ~ignored & ~bad
    rows = np.nonzero(ok)[0]
    loss[rows] = lse[rows] - (1.0 - eps) * x[rows, y[rows]] - eps * x[rows].mean(axis=1)
    loss[bad] = np.nan
    return loss.astype(np.float32), lse.astype(np.float32)


def cross_entropy_bwd(logits, targets, smoothing, ignore_index, grad_scale):
    """Gradient of sum_t grad_scale * loss_t with respect to the logits:
    grad_scale (softmax(x) - (1 - eps) onehot(y) - eps / V), zero on ignored
    rows, NaN on rows with an out-of-range target; rounded once to fp16.
    Parity: pinned by tests (torch autograd of cross_entropy in float64).
    """
    x, y, eps, lse, ignored, bad = _xent_rows(logits, targets, smoothing, ignore_index)
    v = x.shape[1]
    with np.errstate(invalid="ignore", over="ignore"):
        g = np.exp(x - lse[:, None]) - eps / v
    ok = ~ignored & ~bad
    rows = np.nonzero(ok)[0]
    g[rows, y[rows]] -= 1.0 - eps
    g[ignored] = 0.0
    g[bad] = np.nan
    return (float(np.float32(grad_scale)) * g).astype(np.float16)


# ----------------------------------------------------------------------------
# Beam-search top-k by hierarchical filtering (HARS; [L10] beam search slides)
# ----------------------------------------------------------------------------


def _rank_keys(c):
    """Unsigned keys monotone in the float32 value: -0 < +0, every NaN largest."""
    u = np.asarray(c, np.float32).view(np.uint32).astype(np.uint64)
    key = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000)
    return np.where(np.isnan(c), np.uint64(0xFFFFFFFF), key).astype(np.uint64)


def beam_candidates(log_probs, beam_scores):
    """c[b, i, v] = log_probs[b, i, v] + beam_scores[b, i], one float32 add.

    Parity: pinned by a hand-computed fixture (tests/golden/
    beam_candidates_fp32.txt: exact sums, ties to even, an absorbed
    addend) and by the full sort, whose candidates come from torch.
    """
    lp = np.asarray(log_probs, np.float32)
    if beam_scores is None:
        return lp.copy()
    return (lp + np.asarray(beam_scores, np.float32)[:, :, None]).astype(np.float32)


def hars_topk(log_probs, beam_scores, k, return_survivors=False):
    """Top-k of each batch element's beam x V candidates, by the pages' steps.

    1. split every beam's V candidates into k groups (contiguous, as even as
       possible) and take each group's maximum;
    2. the smallest of the k maxima, R_i, is reached by at least k of the
       beam's candidates; R = max over beams of R_i (the pages leave the
       combination across beams open: any beam's R_i bounds the k-th best
       candidate from below, the largest is the tightest);
    3. keep the candidates >= R (the pages say "greater than"; a group
       maximum equal to R can itself be among the best k, so equality must be
       kept) and sort them: value descending, ties by the smaller flat index
       i * V + v.
    A beam with fewer than k candidates gives no bound.
    log_probs float32 [batch, beam, V]; beam_scores float32 [batch, beam] or
    None.  Returns (scores float32 [batch, k], flat ids int32 [batch, k]) and,
    with return_survivors, the survivor count per batch element.
    Parity: pinned by tests (a full sort of every candidate gives the same
    top-k; the bound holds; a beam 2, vocab 8 case keeps 5 of 16).
    """
    c = beam_candidates(log_probs, beam_scores)
    batch, beam, v = c.shape
    if not 1 <= k <= beam * v:
        raise ValueError("need 1 <= k <= beam * V")
    keys = _rank_keys(c)
    scores = np.empty((batch, k), np.float32)
    ids = np.empty((batch, k), np.int32)
    survivors = np.empty(batch, np.int64)
    for b in range(batch):
        r = np.uint64(0)
        for i in range(beam):
            if v >= k:
                maxima = [g.max() for g in np.array_split(keys[b, i], k)]
                r = max(r, min(maxima))
        flat = keys[b].reshape(-1)
        kept = np.nonzero(flat >= r)[0]
        survivors[b] = kept.size
        order = np.lexsort((kept, -flat[kept].astype(np.int64)))      # key descending, index ascending
        best = kept[order[:k]]
        ids[b] = best
        scores[b] = c[b].reshape(-1)[best]
    if return_survivors:
        return scores, ids, survivors
    return scores, ids


# ----------------------------------------------------------------------------
# LayerNorm ([L10] technique 2, slides 21-22)
# ----------------------------------------------------------------------------


def layernorm_fwd(x, gamma, beta, eps):
    """Two-pass LayerNorm over the last axis.

    mean = sum(x) / H;  var = sum((x - mean)^2) / H  (biased);
    rstd = 1 / sqrt(var + eps);  y = (x - mean) * rstd * gamma + beta.
    The pages write sigma = sqrt(E[x^2] - E[x]^2) without eps; eps is read as
    going inside the root, as in every training LayerNorm.
    Returns (y fp16 [rows, H], mean fp32 [rows], rstd fp32 [rows]).
    Parity: pinned by tests (constant row gives beta; the row (+a, -a, ...)
    gives +-a / sqrt(a^2 + eps); torch.nn.functional.layer_norm in fp64;
    one-pass and two-pass variance agree in fp64).
    """
    x64 = np.asarray(x, dtype=np.float64)
    g64 = np.asarray(gamma, dtype=np.float64)
    b64 = np.asarray(beta, dtype=np.float64)
    eps64 = float(np.float32(eps))
    h = x64.shape[-1]
    mean = x64.sum(axis=-1) / h
    centered = x64 - mean[:, None]
    var = (centered * centered).sum(axis=-1) / h
    rstd = 1.0 / np.sqrt(var + eps64)
    y = centered * rstd[:, None] * g64[None, :] + b64[None, :]
    return y.astype(np.float16), mean.astype(np.float32), rstd.astype(np.float32)


def bias_dropout_residual_layernorm(x, bias, residual, gamma, beta, p, seed, offset, bits, eps):
    """z = residual + Dropout(x + bias), rounded to fp16, then LayerNorm of z.

    The sub-layer output block of a post-LN Transformer layer ([LS2]
    sec. 2.1.1: bias, dropout and residual add, then layer normalisation;
    [L10] technique 1 fuses such neighbours).  The LayerNorm reads the stored
    fp16 z, exactly as the two operators called one after the other.
    Returns (z fp16, y fp16, mean fp32, rstd fp32).
    Parity: the composition of bias_dropout_residual and layernorm_fwd, each
    pinned on its own; pinned as a whole by tests against torch's float64
    layer_norm of the fp16 sum (and constant residual rows giving beta).
    """
    z = bias_dropout_residual(x, bias, residual, p, seed, offset, bits)
    y, mean, rstd = layernorm_fwd(z, gamma, beta, eps)
    return z, y, mean, rstd


def layernorm_bwd(dy, x, gamma, mean, rstd):
    """LayerNorm backward given the saved row statistics.

    With xhat = (x - mean) * rstd and g = gamma * dy (per row of length H):
      dx     = rstd * (g - sum(g)/H - xhat * sum(g * xhat)/H)
      dgamma = sum over rows of dy * xhat
      dbeta  = sum over rows of dy
    This is the derivative of layernorm_fwd written out directly; [L10]
    slide 22 regroups the same expression into two row sums that can be
    reduced together.
    Returns (dx fp16 [rows, H], dgamma fp16 [H], dbeta fp16 [H]).
    Parity: pinned by tests (central finite differences through
    layernorm_fwd; torch autograd in fp64; per-row invariants sum(dx) = 0 and
    sum(dx * xhat) = 0).
    """
    dy64 = np.asarray(dy, dtype=np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    g64 = np.asarray(gamma, dtype=np.float64)
    mu = np.asarray(mean, dtype=np.float64)[:, None]
    rs = np.asarray(rstd, dtype=np.float64)[:, None]
    h = x64.shape[-1]
    xhat = (x64 - mu) * rs
    g = g64[None, :] * dy64
    sum_g = g.sum(axis=-1, keepdims=True)
    sum_gx = (g * xhat).sum(axis=-1, keepdims=True)
    dx = rs * (g - sum_g / h - xhat * sum_gx / h)
    dgamma = (dy64 * xhat).sum(axis=0)
    dbeta = dy64.sum(axis=0)
    return dx.astype(np.float16), dgamma.astype(np.float16), dbeta.astype(np.float16)


# ----------------------------------------------------------------------------
# Softmax ([L10] slides 23-26)
# ----------------------------------------------------------------------------


def softmax_valid(batch, heads, q_len, k_len, key_lengths=None, causal=False):
    """Boolean [batch, heads, q_len, k_len] mask of the keys a row may attend to.

    Key j of query row i in sequence b is valid iff j < key_lengths[b] (when
    given; values are clamped into [0, k_len]) and, when causal, j <= i.
    Padding masks only keys; padded query rows still attend to the valid keys.
    """
    j = np.arange(k_len)[None, None, None, :]
    valid = np.ones((batch, heads, q_len, k_len), dtype=bool)
    if key_lengths is not None:
        lens = np.clip(np.asarray(key_lengths, dtype=np.int64), 0, k_len)
        valid &= j < lens[:, None, None, None]
    if causal:
        i = np.arange(q_len)[None, None, :, None]
        valid &= j <= i
    return valid


def softmax_fwd(x, key_lengths=None, causal=False):
    """Masked row softmax over the last axis, two passes.

    x: fp16 [batch, heads, q_len, k_len].  For each row, m = max of the valid
    entries, e_j = exp(x_j - m) on valid entries and 0 elsewhere,
    y = e / sum(e).  A row with no valid entry is all zeros.
    Returns y fp16 of x's shape.
    Parity: pinned by tests (scipy.special.softmax; rows sum to one; the
    online max/normaliser recurrence of [CS336] sec. 6.2 agrees; masked
    entries exactly zero; constant row gives 1/|valid|).
    """
    x64 = np.asarray(x, dtype=np.float64)
    b, h, q, k = x64.shape
    valid = softmax_valid(b, h, q, k, key_lengths, causal)
    masked = np.where(valid, x64, -np.inf)
    m = masked.max(axis=-1, keepdims=True)
    # A row whose valid entries are all -inf (or that has none) normalises to
    # zeros; +inf or NaN inputs give NaN rows, as exp(x - m) / sum does.
    m = np.where(m == -np.inf, 0.0, m)
    e = np.where(valid, np.exp(masked - m), 0.0)
    s = e.sum(axis=-1, keepdims=True)
    y = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
    return y.astype(np.float16)


def softmax_bwd(y, dy):
    """Softmax backward from the stored output: dx = y * (dy - sum(y * dy)).

    y, dy: fp16 [..., k_len]; the sum runs over the last axis.  Masked entries
    have y = 0 and therefore dx = 0, so no mask argument is needed.
    Returns dx fp16.
    Parity: pinned by tests (finite differences through softmax_fwd in fp64;
    rows of dx sum to zero; constant dy gives dx = 0).
    """
    y64 = np.asarray(y, dtype=np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    dot = (y64 * dy64).sum(axis=-1, keepdims=True)
    return (y64 * (dy64 - dot)).astype(np.float16)


# ----------------------------------------------------------------------------
# Embedding ([LS2] sec. 2.1.2)
# ----------------------------------------------------------------------------


def embedding_fwd(ids, tok_emb, pos_emb, scale, p, seed, offset, bits):
    """out[t] = Dropout(s * E[ids_t] + P[t mod L]), rounded once to fp16.

    ids: int32 [batch, L]; tok_emb E: fp16 [V, H]; pos_emb P: fp16
    [max_pos, H] with max_pos >= L; scale s (e.g. sqrt(d_model)).
    Token t = b * L + l sits at position l.  Element (t, c) uses the flat index
    t * H + c for its dropout decision.  A token id outside [0, V) yields a
    row of NaN (its table row is never read).
    Returns fp16 [batch * L, H].
    Parity: pinned by tests (p = 0 and P = 0 give the exact gather times a
    power-of-two scale; torch.nn.functional.embedding).
    """
    ids = np.asarray(ids, dtype=np.int64)
    e64 = np.asarray(tok_emb, dtype=np.float64)
    p64 = np.asarray(pos_emb, dtype=np.float64)
    batch, seq = ids.shape
    vocab, hidden = e64.shape
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < vocab)
    rows = e64[np.where(ok, flat, 0)]
    pos = np.tile(np.arange(seq), batch)
    s = float(np.float32(scale))
    val = s * rows + p64[pos]
    val = val * _masked_scale(val.shape, p, seed, offset, bits)
    val[~ok] = np.nan
    return val.astype(np.float16)


def embedding_bwd(ids, dy, vocab, scale, p, seed, offset, bits, grad_in=None):
    """grad E[w] += s * sum over tokens t with ids_t = w of m_t * dy_t.

    m_t is the forward's mask (keep times the inverted scale), regenerated
    from (seed, offset).  ids: int32 [batch, L]; dy: fp16 [batch * L, H].
    ``grad_in`` (fp32 [V, H]) is the accumulator the caller passes; None means
    it starts at zero.  Tokens whose id lies outside [0, V) contribute
    nothing.  The sum is taken in float64 and rounded once to fp32.
    Returns fp32 [V, H].
    Parity: pinned by tests (torch autograd through an fp64 embedding lookup;
    an id that occurs once gives exactly s * m * dy; the column sums of the
    gradient equal s * sum of m * dy).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    dy64 = np.asarray(dy, dtype=np.float64)
    hidden = dy64.shape[-1]
    dy64 = dy64.reshape(-1, hidden)
    s = float(np.float32(scale))
    contrib = s * dy64 * _masked_scale(dy64.shape, p, seed, offset, bits)
    acc = np.zeros((vocab, hidden), dtype=np.float64)
    if grad_in is not None:
        acc += np.asarray(grad_in, dtype=np.float64)
    ok = (ids >= 0) & (ids < vocab)
    np.add.at(acc, ids[ok], contrib[ok])
    return acc.astype(np.float32)


# ----------------------------------------------------------------------------
# Mixed-precision Adam over the fp16 workspace ([L10] slide 29; [LS2] sec. 2.3)
# ----------------------------------------------------------------------------


def adam_workspace_step(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps,
                        weight_decay, step, grad_scale=1.0, decoupled_wd=True):
    """One Adam step on fp16 parameters and gradients with fp32 moments.

    The trainer of [LS2] sec. 2.3 keeps parameters and gradients only in
    fp16 and widens them on the fly; no fp32 master copy exists.  With
    t = step (1-based), g = grad / grad_scale (loss scaling, [CS336] 3.2):
      (L2 form only) g += wd * p
      m = beta1 * m + (1 - beta1) * g
      v = beta2 * v + (1 - beta2) * g^2
      update = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
      (decoupled form, AdamW) update += wd * p
      p = p - lr * update
    The moments are rounded to fp32 when stored and the stored values feed
    the update; the new parameter is rounded once to fp16.  Hyper-parameters
    are taken as the float32 values the caller passes.
    Returns (param fp16, exp_avg fp32, exp_avg_sq fp32).
    Parity: pinned by tests (step-1 closed form; zero gradient gives
    p * (1 - lr * wd); torch.optim.AdamW / Adam in fp64 without the storage
    roundings).
    """
    f = lambda v: float(np.float32(v))  # noqa: E731
    lr, beta1, beta2, eps, wd, gs = map(f, (lr, beta1, beta2, eps, weight_decay, grad_scale))
    t = int(step)
    if t < 1:
        raise ValueError("step is 1-based")
    p64 = np.asarray(param, dtype=np.float64)
    g64 = np.asarray(grad, dtype=np.float64) / gs
    m64 = np.asarray(exp_avg, dtype=np.float64)
    v64 = np.asarray(exp_avg_sq, dtype=np.float64)
    if not decoupled_wd:
        g64 = g64 + wd * p64
    m_new = (beta1 * m64 + (1.0 - beta1) * g64).astype(np.float32)
    v_new = (beta2 * v64 + (1.0 - beta2) * g64 * g64).astype(np.float32)
    m_hat = m_new.astype(np.float64) / (1.0 - beta1 ** t)
    v_hat = v_new.astype(np.float64) / (1.0 - beta2 ** t)
    update = m_hat / (np.sqrt(v_hat) + eps)
    if decoupled_wd:
        update = update + wd * p64
    p_new = (p64 - lr * update).astype(np.float16)
    return p_new, m_new, v_new
