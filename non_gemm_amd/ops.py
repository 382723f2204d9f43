"""Torch-tensor front end of the ls_mi355 C ABI.

Argument marshalling only: every function checks device, dtype, contiguity
and shapes, passes raw device pointers and the current HIP stream to the
library, and raises LsError on a non-zero status.  All arithmetic runs in the
library's HIP kernels; nothing here computes on the host.
"""

import ctypes

import torch

from ._lib import check, load

_F16 = torch.float16
_F32 = torch.float32


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _dev(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("ls_mi355 ops take device (cuda/HIP) tensors")
        if not t.is_contiguous():
            raise ValueError("ls_mi355 ops take contiguous tensors")


def _dtype(t, dt, what):
    if t.dtype != dt:
        raise TypeError(f"{what} must be {dt}, got {t.dtype}")


def _rows_cols(x):
    if x.dim() < 1:
        raise ValueError("need at least one dimension")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    return rows, cols


def bias_dropout_residual(x, bias, residual, p, seed, offset, out=None):
    """out = residual + Dropout(x + bias); x, residual [..., H] fp16, bias [H]."""
    _dev(x, bias, residual, out)
    for t, n in ((x, "x"), (bias, "bias"), (residual, "residual")):
        _dtype(t, _F16, n)
    if residual.shape != x.shape or bias.shape != (x.shape[-1],):
        raise ValueError("shape mismatch")
    out = torch.empty_like(x) if out is None else out
    rows, cols = _rows_cols(x)
    check("ls_bias_dropout_residual", load().ls_bias_dropout_residual(
        _ptr(out), _ptr(x), _ptr(bias), _ptr(residual), rows, cols, float(p), int(seed), int(offset), _stream()))
    return out


def bias_relu_dropout(x, bias, p, seed, offset, out=None):
    """out = Dropout(ReLU(x + bias)); x [..., F] fp16, bias [F]."""
    _dev(x, bias, out)
    _dtype(x, _F16, "x")
    _dtype(bias, _F16, "bias")
    if bias.shape != (x.shape[-1],):
        raise ValueError("shape mismatch")
    out = torch.empty_like(x) if out is None else out
    rows, cols = _rows_cols(x)
    check("ls_bias_relu_dropout", load().ls_bias_relu_dropout(
        _ptr(out), _ptr(x), _ptr(bias), rows, cols, float(p), int(seed), int(offset), _stream()))
    return out


def elementwise_bwd_workspace_bytes(rows, cols):
    return int(load().ls_elementwise_bwd_workspace_bytes(int(rows), int(cols)))


def _ew_bwd_buffers(dy, dx, dbias, workspace):
    rows, cols = _rows_cols(dy)
    dx = torch.empty_like(dy) if dx is None else dx
    dbias = torch.empty(cols, dtype=_F16, device=dy.device) if dbias is None else dbias
    if workspace is None:
        workspace = torch.empty(max(elementwise_bwd_workspace_bytes(rows, cols), 16), dtype=torch.uint8,
                                device=dy.device)
    return rows, cols, dx, dbias, workspace


def bias_dropout_residual_bwd(dy, p, seed, offset, dx=None, dbias=None, workspace=None):
    """Backward of bias_dropout_residual: returns (dx fp16, dbias fp16 [H]);
    the residual's gradient is dy itself.  seed and offset are the forward's."""
    _dev(dy, dx, dbias, workspace)
    _dtype(dy, _F16, "dy")
    rows, cols, dx, dbias, workspace = _ew_bwd_buffers(dy, dx, dbias, workspace)
    check("ls_bias_dropout_residual_bwd", load().ls_bias_dropout_residual_bwd(
        _ptr(dx), _ptr(dbias), _ptr(dy), rows, cols, float(p), int(seed), int(offset), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return dx, dbias


def bias_relu_dropout_bwd(dy, out, p, dx=None, dbias=None, workspace=None):
    """Backward of bias_relu_dropout from its output: returns (dx fp16, dbias fp16 [F])."""
    _dev(dy, out, dx, dbias, workspace)
    _dtype(dy, _F16, "dy")
    _dtype(out, _F16, "out")
    if out.shape != dy.shape:
        raise ValueError("shape mismatch")
    rows, cols, dx, dbias, workspace = _ew_bwd_buffers(dy, dx, dbias, workspace)
    check("ls_bias_relu_dropout_bwd", load().ls_bias_relu_dropout_bwd(
        _ptr(dx), _ptr(dbias), _ptr(dy), _ptr(out), rows, cols, float(p), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return dx, dbias


def bias_qkv_split(qkv, bias, batch, seq_len, heads, out=None):
    """qkv [batch*seq_len, 3H] fp16 + bias [3H] -> [3, batch, heads, seq_len, head_dim]."""
    _dev(qkv, bias, out)
    _dtype(qkv, _F16, "qkv")
    _dtype(bias, _F16, "bias")
    tokens, cols = _rows_cols(qkv)
    if tokens != batch * seq_len or cols % (3 * heads) or bias.shape != (cols,):
        raise ValueError("shape mismatch")
    d = cols // (3 * heads)
    out = torch.empty((3, batch, heads, seq_len, d), dtype=_F16, device=qkv.device) if out is None else out
    check("ls_bias_qkv_split", load().ls_bias_qkv_split(
        _ptr(out), _ptr(qkv), _ptr(bias), int(batch), int(seq_len), int(heads), int(d), _stream()))
    return out


def bias_qkv_split_bwd(dout, dqkv=None, dbias=None, workspace=None):
    """dout [3, batch, heads, seq_len, head_dim] -> (dqkv [batch*seq_len, 3H], dbias [3H])."""
    _dev(dout, dqkv, dbias, workspace)
    _dtype(dout, _F16, "dout")
    if dout.dim() != 5 or dout.shape[0] != 3:
        raise ValueError("dout must be [3, batch, heads, seq_len, head_dim]")
    _, b, h, l, d = dout.shape
    tokens, cols = b * l, 3 * h * d
    dqkv = torch.empty((tokens, cols), dtype=_F16, device=dout.device) if dqkv is None else dqkv
    dbias = torch.empty(cols, dtype=_F16, device=dout.device) if dbias is None else dbias
    if workspace is None:
        workspace = torch.empty(max(elementwise_bwd_workspace_bytes(tokens, cols), 16), dtype=torch.uint8,
                                device=dout.device)
    check("ls_bias_qkv_split_bwd", load().ls_bias_qkv_split_bwd(
        _ptr(dqkv), _ptr(dbias), _ptr(dout), int(b), int(l), int(h), int(d), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return dqkv, dbias


def cross_entropy_fwd(logits, targets, smoothing=0.0, ignore_index=-1, loss=None, lse=None):
    """logits [rows, vocab] fp16, targets int32 [rows] -> (loss fp32 [rows], lse fp32 [rows])."""
    _dev(logits, targets, loss, lse)
    _dtype(logits, _F16, "logits")
    _dtype(targets, torch.int32, "targets")
    rows, vocab = _rows_cols(logits)
    if targets.numel() != rows:
        raise ValueError("one target per row")
    loss = torch.empty(rows, dtype=_F32, device=logits.device) if loss is None else loss
    lse = torch.empty(rows, dtype=_F32, device=logits.device) if lse is None else lse
    check("ls_cross_entropy_fwd", load().ls_cross_entropy_fwd(
        _ptr(loss), _ptr(lse), _ptr(logits), _ptr(targets), rows, vocab, float(smoothing), int(ignore_index),
        _stream()))
    return loss, lse


def cross_entropy_bwd(logits, targets, lse, smoothing=0.0, ignore_index=-1, grad_scale=1.0, dlogits=None):
    """Gradient of sum_t grad_scale * loss[t] with respect to the logits (fp16, logits' shape)."""
    _dev(logits, targets, lse, dlogits)
    _dtype(logits, _F16, "logits")
    _dtype(targets, torch.int32, "targets")
    _dtype(lse, _F32, "lse")
    rows, vocab = _rows_cols(logits)
    if targets.numel() != rows or lse.numel() != rows:
        raise ValueError("one target and one lse per row")
    dlogits = torch.empty_like(logits) if dlogits is None else dlogits
    check("ls_cross_entropy_bwd", load().ls_cross_entropy_bwd(
        _ptr(dlogits), _ptr(logits), _ptr(targets), _ptr(lse), rows, vocab, float(smoothing), int(ignore_index),
        float(grad_scale), _stream()))
    return dlogits


def beam_topk(log_probs, k, beam_scores=None, top_scores=None, top_ids=None, workspace=None):
    """log_probs fp32 [batch, beam, vocab] (+ beam_scores fp32 [batch, beam]) ->
    (top_scores fp32 [batch, k], top_ids int32 [batch, k], flat i * vocab + v)."""
    _dev(log_probs, beam_scores, top_scores, top_ids, workspace)
    _dtype(log_probs, _F32, "log_probs")
    if log_probs.dim() != 3:
        raise ValueError("log_probs must be [batch, beam, vocab]")
    batch, beam, vocab = log_probs.shape
    if beam_scores is not None:
        _dtype(beam_scores, _F32, "beam_scores")
        if beam_scores.shape != (batch, beam):
            raise ValueError("beam_scores must be [batch, beam]")
    top_scores = torch.empty((batch, k), dtype=_F32, device=log_probs.device) if top_scores is None else top_scores
    top_ids = torch.empty((batch, k), dtype=torch.int32, device=log_probs.device) if top_ids is None else top_ids
    lib = load()
    if workspace is None:
        need = int(lib.ls_beam_topk_workspace_bytes(batch, beam, int(k)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=log_probs.device)
    check("ls_beam_topk", lib.ls_beam_topk(
        _ptr(top_scores), _ptr(top_ids), _ptr(log_probs), _ptr(beam_scores), batch, beam, vocab, int(k),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return top_scores, top_ids


def layernorm_fwd(x, gamma, beta, eps, y=None, mean=None, rstd=None):
    """Returns (y fp16, mean fp32 [rows], rstd fp32 [rows])."""
    _dev(x, gamma, beta, y, mean, rstd)
    for t, n in ((x, "x"), (gamma, "gamma"), (beta, "beta")):
        _dtype(t, _F16, n)
    rows, h = _rows_cols(x)
    if gamma.shape != (h,) or beta.shape != (h,):
        raise ValueError("shape mismatch")
    y = torch.empty_like(x) if y is None else y
    mean = torch.empty(rows, dtype=_F32, device=x.device) if mean is None else mean
    rstd = torch.empty(rows, dtype=_F32, device=x.device) if rstd is None else rstd
    check("ls_layernorm_fwd", load().ls_layernorm_fwd(
        _ptr(y), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(gamma), _ptr(beta), rows, h, float(eps), _stream()))
    return y, mean, rstd


def bias_dropout_residual_layernorm(x, bias, residual, gamma, beta, p, seed, offset, eps, z=None, y=None,
                                    mean=None, rstd=None):
    """z = residual + Dropout(x + bias) and its LayerNorm, one launch.
    Returns (z fp16, y fp16, mean fp32 [rows], rstd fp32 [rows])."""
    _dev(x, bias, residual, gamma, beta, z, y, mean, rstd)
    for t, n in ((x, "x"), (bias, "bias"), (residual, "residual"), (gamma, "gamma"), (beta, "beta")):
        _dtype(t, _F16, n)
    rows, h = _rows_cols(x)
    if residual.shape != x.shape or bias.shape != (h,) or gamma.shape != (h,) or beta.shape != (h,):
        raise ValueError("shape mismatch")
    z = torch.empty_like(x) if z is None else z
    y = torch.empty_like(x) if y is None else y
    mean = torch.empty(rows, dtype=_F32, device=x.device) if mean is None else mean
    rstd = torch.empty(rows, dtype=_F32, device=x.device) if rstd is None else rstd
    check("ls_bias_dropout_residual_layernorm", load().ls_bias_dropout_residual_layernorm(
        _ptr(z), _ptr(y), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(bias), _ptr(residual), _ptr(gamma), _ptr(beta),
        rows, h, float(p), int(seed), int(offset), float(eps), _stream()))
    return z, y, mean, rstd


def layernorm_bwd_workspace_bytes(rows, hidden):
    return int(load().ls_layernorm_bwd_workspace_bytes(int(rows), int(hidden)))


def layernorm_bwd(dy, x, gamma, mean, rstd, dx=None, dgamma=None, dbeta=None, workspace=None):
    """Returns (dx fp16, dgamma fp16 [H], dbeta fp16 [H])."""
    _dev(dy, x, gamma, mean, rstd, dx, dgamma, dbeta, workspace)
    rows, h = _rows_cols(x)
    if dy.shape != x.shape or gamma.shape != (h,) or mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("shape mismatch")
    dx = torch.empty_like(x) if dx is None else dx
    dgamma = torch.empty(h, dtype=_F16, device=x.device) if dgamma is None else dgamma
    dbeta = torch.empty(h, dtype=_F16, device=x.device) if dbeta is None else dbeta
    need = layernorm_bwd_workspace_bytes(rows, h)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    check("ls_layernorm_bwd", load().ls_layernorm_bwd(
        _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd),
        rows, h, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return dx, dgamma, dbeta


def layernorm_bwd_input(dy, x, gamma, mean, rstd, workspace, dx=None):
    """First half of layernorm_bwd: dx, and the dgamma / dbeta partials in
    `workspace` (uint8, at least layernorm_bwd_workspace_bytes).  Returns dx."""
    _dev(dy, x, gamma, mean, rstd, dx, workspace)
    rows, h = _rows_cols(x)
    if dy.shape != x.shape or gamma.shape != (h,) or mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("shape mismatch")
    dx = torch.empty_like(x) if dx is None else dx
    check("ls_layernorm_bwd_input", load().ls_layernorm_bwd_input(
        _ptr(dx), _ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), rows, h, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return dx


def layernorm_bwd_params(rows, hidden, workspace, dgamma=None, dbeta=None, device="cuda"):
    """Second half of layernorm_bwd: dgamma, dbeta from the partials of the
    matching layernorm_bwd_input call.  Returns (dgamma, dbeta)."""
    _dev(workspace, dgamma, dbeta)
    dgamma = torch.empty(hidden, dtype=_F16, device=device) if dgamma is None else dgamma
    dbeta = torch.empty(hidden, dtype=_F16, device=device) if dbeta is None else dbeta
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("ls_layernorm_bwd_params", load().ls_layernorm_bwd_params(
        _ptr(dgamma), _ptr(dbeta), int(rows), int(hidden), _ptr(workspace), nbytes, _stream()))
    return dgamma, dbeta


def layernorm_bwd_params_batched(jobs, device="cuda"):
    """layernorm_bwd_params for several LayerNorms in one launch.  jobs: a
    list of (rows, hidden, workspace, dgamma, dbeta), dgamma / dbeta None to
    allocate.  Returns [(dgamma, dbeta), ...] in job order."""
    n = len(jobs)
    outs = []
    for rows, hidden, ws, dg, db in jobs:
        _dev(ws, dg, db)
        dg = torch.empty(hidden, dtype=_F16, device=device) if dg is None else dg
        db = torch.empty(hidden, dtype=_F16, device=device) if db is None else db
        outs.append((dg, db, ws))
    ptrs = ctypes.c_void_p * max(n, 1)
    i64s = ctypes.c_int64 * max(n, 1)
    sizes = ctypes.c_size_t * max(n, 1)
    dgs = ptrs(*[_ptr(o[0]) for o in outs])
    dbs = ptrs(*[_ptr(o[1]) for o in outs])
    wss = ptrs(*[_ptr(o[2]) for o in outs])
    rows = i64s(*[int(j[0]) for j in jobs])
    hid = i64s(*[int(j[1]) for j in jobs])
    nb = sizes(*[0 if o[2] is None else o[2].numel() * o[2].element_size() for o in outs])
    check("ls_layernorm_bwd_params_batched", load().ls_layernorm_bwd_params_batched(
        n, dgs, dbs, rows, hid, wss, nb, _stream()))
    return [(o[0], o[1]) for o in outs]


def softmax_fwd(x, key_lengths=None, causal=False, y=None):
    """x [batch, heads, q_len, k_len] fp16; key_lengths int32 [batch] or None."""
    _dev(x, key_lengths, y)
    _dtype(x, _F16, "x")
    if x.dim() != 4:
        raise ValueError("x must be [batch, heads, q_len, k_len]")
    b, h, q, k = x.shape
    if key_lengths is not None:
        _dtype(key_lengths, torch.int32, "key_lengths")
        if key_lengths.numel() != b:
            raise ValueError("key_lengths must have one entry per sequence")
    y = torch.empty_like(x) if y is None else y
    check("ls_softmax_fwd", load().ls_softmax_fwd(
        _ptr(y), _ptr(x), b, h, q, k, _ptr(key_lengths), int(bool(causal)), _stream()))
    return y


def softmax_bwd(y, dy, dx=None):
    """dx = y * (dy - sum(y * dy)) over the last axis."""
    _dev(y, dy, dx)
    _dtype(y, _F16, "y")
    _dtype(dy, _F16, "dy")
    if dy.shape != y.shape:
        raise ValueError("shape mismatch")
    dx = torch.empty_like(y) if dx is None else dx
    rows, k = _rows_cols(y)
    check("ls_softmax_bwd", load().ls_softmax_bwd(_ptr(dx), _ptr(y), _ptr(dy), rows, k, _stream()))
    return dx


def embedding_fwd(ids, tok_emb, pos_emb, scale, p, seed, offset, out=None):
    """ids int32 [batch, L]; tok_emb fp16 [V, H]; pos_emb fp16 [max_pos, H]."""
    _dev(ids, tok_emb, pos_emb, out)
    _dtype(ids, torch.int32, "ids")
    _dtype(tok_emb, _F16, "tok_emb")
    _dtype(pos_emb, _F16, "pos_emb")
    b, l = ids.shape
    v, h = tok_emb.shape
    out = torch.empty((b * l, h), dtype=_F16, device=ids.device) if out is None else out
    check("ls_embedding_fwd", load().ls_embedding_fwd(
        _ptr(out), _ptr(ids), _ptr(tok_emb), _ptr(pos_emb), b, l, h, v, pos_emb.shape[0],
        float(scale), float(p), int(seed), int(offset), _stream()))
    return out


def embedding_bwd(ids, dy, grad_tok_emb, scale, p, seed, offset, zero_first=True):
    """grad_tok_emb fp32 [V, H] (+)= scale * sum of masked dy rows per id."""
    _dev(ids, dy, grad_tok_emb)
    _dtype(ids, torch.int32, "ids")
    _dtype(dy, _F16, "dy")
    _dtype(grad_tok_emb, _F32, "grad_tok_emb")
    b, l = ids.shape
    v, h = grad_tok_emb.shape
    if dy.numel() != b * l * h:
        raise ValueError("dy must be [batch * L, H]")
    check("ls_embedding_bwd", load().ls_embedding_bwd(
        _ptr(grad_tok_emb), _ptr(ids), _ptr(dy), b, l, h, v, float(scale), float(p), int(seed),
        int(offset), int(bool(zero_first)), _stream()))
    return grad_tok_emb


def adam_workspace_step(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay,
                        step, grad_scale=1.0, decoupled_wd=True):
    """One in-place Adam step over flat fp16 param/grad and fp32 moments."""
    _dev(param, grad, exp_avg, exp_avg_sq)
    _dtype(param, _F16, "param")
    _dtype(grad, _F16, "grad")
    _dtype(exp_avg, _F32, "exp_avg")
    _dtype(exp_avg_sq, _F32, "exp_avg_sq")
    n = param.numel()
    if grad.numel() != n or exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("workspace tensors must have equal length")
    check("ls_adam_workspace_step", load().ls_adam_workspace_step(
        _ptr(param), _ptr(grad), _ptr(exp_avg), _ptr(exp_avg_sq), n, float(lr), float(beta1),
        float(beta2), float(eps), float(weight_decay), int(step), float(grad_scale),
        int(bool(decoupled_wd)), _stream()))


def dropout_mask(n, p, seed, offset, device="cuda"):
    """uint8 [n]: 1 where the dropout kernels keep element i, 0 where they drop it."""
    keep = torch.empty(int(n), dtype=torch.uint8, device=device)
    check("ls_dropout_mask", load().ls_dropout_mask(_ptr(keep), int(n), float(p), int(seed), int(offset), _stream()))
    return keep
