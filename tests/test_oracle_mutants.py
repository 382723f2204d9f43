"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in an oracle function -- a dropped term,
a wrong sign, a wrong index or order, a transposed mask -- by swapping a
faulty copy into the ``oracle`` package for the duration of the case, then
runs the pin tests of that function from test_oracle_ops.py and
test_golden.py.  At least one of them must fail; a mistake no pin notices
would be a hole in the pins.  The faulty copies live only here.
"""
import numpy as np
import pytest

import oracle
import test_golden as golden
import test_oracle_ops as pins
from oracle.ops import dropout_keep, dropout_scale


def _ms(shape, p, seed, offset, bits, scaled=True):
    n = int(np.prod(shape))
    keep = dropout_keep(n, p, seed, offset, bits).astype(np.float64)
    return (keep * (dropout_scale(p, bits) if scaled else 1.0)).reshape(shape)


# ---------------------------------------------------------------- mistakes --

def bdr_unscaled(x, bias, residual, p, seed, offset, bits):
    """Forgets the inverted-dropout scale 1 / (1 - p)."""
    x64, b64, r64 = (np.asarray(a, np.float64) for a in (x, bias, residual))
    return (r64 + _ms(x64.shape, p, seed, offset, bits, scaled=False) * (x64 + b64)).astype(np.float16)


def bdr_bias_after_dropout(x, bias, residual, p, seed, offset, bits):
    """Adds the bias after the dropout instead of before it."""
    x64, b64, r64 = (np.asarray(a, np.float64) for a in (x, bias, residual))
    return (r64 + _ms(x64.shape, p, seed, offset, bits) * x64 + b64).astype(np.float16)


def brd_relu_before_bias(x, bias, p, seed, offset, bits):
    """Applies the ReLU before adding the bias."""
    x64, b64 = np.asarray(x, np.float64), np.asarray(bias, np.float64)
    return (_ms(x64.shape, p, seed, offset, bits) * (np.maximum(x64, 0.0) + b64)).astype(np.float16)


def ln_fwd_unbiased(x, gamma, beta, eps):
    """Divides the variance by H - 1."""
    x64, g64, b64 = (np.asarray(a, np.float64) for a in (x, gamma, beta))
    h = x64.shape[-1]
    mean = x64.mean(axis=-1)
    c = x64 - mean[:, None]
    var = (c * c).sum(axis=-1) / (h - 1)
    rstd = 1.0 / np.sqrt(var + float(np.float32(eps)))
    return (c * rstd[:, None] * g64 + b64).astype(np.float16), mean.astype(np.float32), rstd.astype(np.float32)


def ln_fwd_eps_outside(x, gamma, beta, eps):
    """Adds eps outside the square root."""
    x64, g64, b64 = (np.asarray(a, np.float64) for a in (x, gamma, beta))
    mean = x64.mean(axis=-1)
    c = x64 - mean[:, None]
    rstd = 1.0 / (np.sqrt((c * c).mean(axis=-1)) + float(np.float32(eps)))
    return (c * rstd[:, None] * g64 + b64).astype(np.float16), mean.astype(np.float32), rstd.astype(np.float32)


def _ln_bwd(dy, x, gamma, mean, rstd, mistake):
    dy64, x64, g64 = (np.asarray(a, np.float64) for a in (dy, x, gamma))
    mu = np.asarray(mean, np.float64)[:, None]
    rs = np.asarray(rstd, np.float64)[:, None]
    h = x64.shape[-1]
    xhat = (x64 - mu) * rs
    g = g64 * dy64
    sum_g = g.sum(axis=-1, keepdims=True)
    sum_gx = (g * xhat).sum(axis=-1, keepdims=True)
    if mistake == "no_mean_term":
        dx = rs * (g - xhat * sum_gx / h)
    elif mistake == "sign":
        dx = rs * (g - sum_g / h + xhat * sum_gx / h)
    else:
        dx = rs * (g - sum_g / h - xhat * sum_gx / h)
    dgamma = (dy64 * (x64 if mistake == "dgamma_raw_x" else xhat)).sum(axis=0)
    dbeta = (g if mistake == "dbeta_gamma" else dy64).sum(axis=0)
    return dx.astype(np.float16), dgamma.astype(np.float16), dbeta.astype(np.float16)


def ln_bwd_no_mean_term(dy, x, gamma, mean, rstd):
    """Drops the - sum(g)/H term of dx."""
    return _ln_bwd(dy, x, gamma, mean, rstd, "no_mean_term")


def ln_bwd_sign(dy, x, gamma, mean, rstd):
    """Flips the sign of the xhat * sum(g xhat)/H term."""
    return _ln_bwd(dy, x, gamma, mean, rstd, "sign")


def ln_bwd_dgamma_raw_x(dy, x, gamma, mean, rstd):
    """Sums dy * x for dgamma instead of dy * xhat."""
    return _ln_bwd(dy, x, gamma, mean, rstd, "dgamma_raw_x")


def ln_bwd_dbeta_gamma(dy, x, gamma, mean, rstd):
    """Sums gamma * dy for dbeta instead of dy."""
    return _ln_bwd(dy, x, gamma, mean, rstd, "dbeta_gamma")


def _softmax(x, key_lengths, causal, mistake):
    x64 = np.asarray(x, np.float64)
    b, h, q, k = x64.shape
    j = np.arange(k)[None, None, None, :]
    i = np.arange(q)[None, None, :, None]
    valid = np.ones(x64.shape, bool)
    if key_lengths is not None:
        lens = np.clip(np.asarray(key_lengths, np.int64), 0, k)[:, None, None, None]
        valid &= (i < lens) if mistake == "mask_queries" else (j < lens)
    if causal:
        valid &= (j < i) if mistake == "causal_strict" else (j <= i)
    masked = np.where(valid, x64, -np.inf)
    m = masked.max(axis=-1, keepdims=True)
    m = np.where(m == -np.inf, 0.0, m)
    e = np.where(valid, np.exp(masked - m), 0.0)
    s = e.sum(axis=-1, keepdims=True)
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0).astype(np.float16)


def softmax_mask_queries(x, key_lengths=None, causal=False):
    """Applies the padding mask to query rows instead of key columns."""
    return _softmax(x, key_lengths, causal, "mask_queries")


def softmax_causal_strict(x, key_lengths=None, causal=False):
    """Causal mask off by one: j < i instead of j <= i."""
    return _softmax(x, key_lengths, causal, "causal_strict")


def softmax_bwd_no_dot(y, dy):
    """Drops the - sum(y dy) term."""
    y64, dy64 = np.asarray(y, np.float64), np.asarray(dy, np.float64)
    return (y64 * dy64).astype(np.float16)


def softmax_bwd_dy_for_y(y, dy):
    """Multiplies by dy where the formula has y."""
    y64, dy64 = np.asarray(y, np.float64), np.asarray(dy, np.float64)
    dot = (y64 * dy64).sum(axis=-1, keepdims=True)
    return (dy64 * (dy64 - dot)).astype(np.float16)


def _emb_fwd(ids, tok_emb, pos_emb, scale, p, seed, offset, bits, mistake):
    ids = np.asarray(ids, np.int64)
    e64, p64 = np.asarray(tok_emb, np.float64), np.asarray(pos_emb, np.float64)
    batch, seq = ids.shape
    vocab = e64.shape[0]
    flat = ids.reshape(-1)
    ok = (flat >= 0) & (flat < vocab)
    rows = e64[np.where(ok, flat, 0)]
    pos = np.repeat(np.arange(batch), seq) % p64.shape[0] if mistake == "position_is_batch" else np.tile(np.arange(seq), batch)
    s = float(np.float32(scale))
    val = rows + s * p64[pos] if mistake == "scale_on_position" else s * rows + p64[pos]
    val = val * _ms(val.shape, p, seed, offset, bits)
    val[~ok] = np.nan
    return val.astype(np.float16)


def emb_fwd_scale_on_position(ids, tok_emb, pos_emb, scale, p, seed, offset, bits):
    """Scales the position row instead of the token row."""
    return _emb_fwd(ids, tok_emb, pos_emb, scale, p, seed, offset, bits, "scale_on_position")


def emb_fwd_position_is_batch(ids, tok_emb, pos_emb, scale, p, seed, offset, bits):
    """Indexes the position table by the sequence instead of the position in it."""
    return _emb_fwd(ids, tok_emb, pos_emb, scale, p, seed, offset, bits, "position_is_batch")


def emb_bwd_no_mask(ids, dy, vocab, scale, p, seed, offset, bits, grad_in=None):
    """Forgets the dropout mask m of the gradient."""
    ids = np.asarray(ids, np.int64).reshape(-1)
    dy64 = np.asarray(dy, np.float64)
    dy64 = dy64.reshape(-1, dy64.shape[-1])
    acc = np.zeros((vocab, dy64.shape[-1]))
    if grad_in is not None:
        acc += np.asarray(grad_in, np.float64)
    ok = (ids >= 0) & (ids < vocab)
    np.add.at(acc, ids[ok], float(np.float32(scale)) * dy64[ok])
    return acc.astype(np.float32)


def _adam(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step, grad_scale, decoupled_wd,
          mistake):
    f = lambda v: float(np.float32(v))  # noqa: E731
    lr, beta1, beta2, eps, wd, gs = map(f, (lr, beta1, beta2, eps, weight_decay, grad_scale))
    t = int(step)
    p64 = np.asarray(param, np.float64)
    g64 = np.asarray(grad, np.float64) / gs
    if not decoupled_wd:
        g64 = g64 + wd * p64
    m = (beta1 * np.asarray(exp_avg, np.float64) + (1 - beta1) * g64).astype(np.float32)
    v = (beta2 * np.asarray(exp_avg_sq, np.float64) + (1 - beta2) * g64 * g64).astype(np.float32)
    if mistake == "no_bias_correction":
        m_hat, v_hat = m.astype(np.float64), v.astype(np.float64)
    else:
        m_hat, v_hat = m / (1 - beta1 ** t), v / (1 - beta2 ** t)
    upd = m_hat / (np.sqrt(v_hat + eps) if mistake == "eps_inside" else np.sqrt(v_hat) + eps)
    if decoupled_wd:
        upd = upd + wd * p64
    return (p64 - lr * upd).astype(np.float16), m, v


def adam_no_bias_correction(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step,
                            grad_scale=1.0, decoupled_wd=True):
    """Leaves out the bias corrections 1 / (1 - beta^t)."""
    return _adam(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step, grad_scale,
                 decoupled_wd, "no_bias_correction")


def adam_eps_inside(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step,
                    grad_scale=1.0, decoupled_wd=True):
    """Adds eps inside the square root."""
    return _adam(param, grad, exp_avg, exp_avg_sq, lr, beta1, beta2, eps, weight_decay, step, grad_scale,
                 decoupled_wd, "eps_inside")


def hars_strict_threshold(log_probs, beam_scores, k, return_survivors=False):
    """Keeps only candidates strictly above the threshold R, then sorts them."""
    c = oracle.beam_candidates(log_probs, beam_scores).astype(np.float64)
    batch, beam, v = c.shape
    bounds = np.linspace(0, v, k + 1).round().astype(int)
    scores = np.empty((batch, k), np.float32)
    ids = np.zeros((batch, k), np.int32)
    surv = np.empty(batch, np.int64)
    for b in range(batch):
        r = max(min(c[b, i, bounds[g]:bounds[g + 1]].max() for g in range(k)) for i in range(beam))
        flat = c[b].reshape(-1)
        kept = np.nonzero(flat > r)[0]
        surv[b] = kept.size
        order = kept[np.lexsort((kept, -flat[kept]))][:k]
        ids[b, :order.size] = order
        scores[b] = np.pad(flat[order], (0, k - order.size), constant_values=-np.inf)
    return (scores, ids, surv) if return_survivors else (scores, ids)


def beam_candidates_sign_flipped(log_probs, beam_scores):
    """Subtracts the beam score instead of adding it."""
    lp = np.asarray(log_probs, np.float32)
    if beam_scores is None:
        return lp.copy()
    return (lp - np.asarray(beam_scores, np.float32)[:, :, None]).astype(np.float32)


def beam_candidates_unrounded(log_probs, beam_scores):
    """Adds in float64 and keeps the sum unrounded."""
    lp = np.asarray(log_probs, np.float64)
    if beam_scores is None:
        return lp.copy()
    return lp + np.asarray(beam_scores, np.float64)[:, :, None]


def fused_ln_of_unrounded_sum(x, bias, residual, gamma, beta, p, seed, offset, bits, eps):
    """Normalises the float64 sum instead of the stored fp16 z."""
    x64, r64 = np.asarray(x, np.float64), np.asarray(residual, np.float64)
    ms = _ms(x64.shape, p, seed, offset, bits)
    z64 = r64 + ms * (x64 + np.asarray(bias, np.float64)[None, :])
    mu = z64.mean(1, keepdims=True)
    var = ((z64 - mu) ** 2).mean(1, keepdims=True)
    rs = 1 / np.sqrt(var + float(np.float32(eps)))
    y = (z64 - mu) * rs * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)
    return z64.astype(np.float16), y.astype(np.float16), mu[:, 0].astype(np.float32), rs[:, 0].astype(np.float32)


def fused_ln_without_residual(x, bias, residual, gamma, beta, p, seed, offset, bits, eps):
    """Drops the residual from the normalised sum (z itself stays right)."""
    z = oracle.bias_dropout_residual(x, bias, residual, p, seed, offset, bits)
    branch = oracle.bias_dropout_residual(x, bias, np.zeros_like(residual), p, seed, offset, bits)
    y, mean, rstd = oracle.layernorm_fwd(branch, gamma, beta, eps)
    return z, y, mean, rstd


def bdr_bwd_no_mask(dy, p, seed, offset, bits):
    """Passes dy through without the dropout mask."""
    dy64 = np.asarray(dy, np.float64)
    return dy64.astype(np.float16), dy64.sum(axis=0).astype(np.float16)


def brd_bwd_gate_on_x(dy, x, bias, p, seed, offset, bits):
    """Gates the gradient on x > 0 instead of x + bias > 0."""
    dy64 = np.asarray(dy, np.float64)
    dx = dy64 * _ms(dy64.shape, p, seed, offset, bits) * (np.asarray(x, np.float64) > 0.0)
    return dx.astype(np.float16), dx.sum(axis=0).astype(np.float16)


def qkv_split_heads_positions_swapped(qkv, bias, batch, seq_len, heads):
    """Lays each part out as [batch, seq_len, heads, d] instead of [batch, heads, seq_len, d]."""
    x = np.asarray(qkv, np.float64) + np.asarray(bias, np.float64)[None, :]
    d = x.shape[1] // (3 * heads)
    y = x.reshape(batch, seq_len, 3, heads, d).transpose(2, 0, 1, 3, 4)
    return np.ascontiguousarray(y).reshape(3, batch, heads, seq_len, d).astype(np.float16)


def _xent(logits, targets, smoothing, ignore_index, mistake):
    x = np.asarray(logits, np.float64)
    y = np.asarray(targets, np.int64).reshape(-1)
    eps = float(np.float32(smoothing))
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    ignored = y == ignore_index
    bad = ~ignored & ((y < 0) | (y >= x.shape[1]))
    ok = ~ignored & ~bad
    rows = np.nonzero(ok)[0]
    loss = np.zeros(x.shape[0])
    v = x.shape[1]
    spread = x[rows].sum(axis=1) / (v - 1) if mistake == "spread_over_v_minus_1" else x[rows].mean(axis=1)
    loss[rows] = lse[rows] - (1.0 - eps) * x[rows, y[rows]] - eps * spread
    loss[bad] = np.nan
    return loss.astype(np.float32), lse.astype(np.float32)


def xent_spread_over_v_minus_1(logits, targets, smoothing, ignore_index):
    """Spreads the smoothing mass over V - 1 classes instead of V."""
    return _xent(logits, targets, smoothing, ignore_index, "spread_over_v_minus_1")


def xent_bwd_no_smoothing_floor(logits, targets, smoothing, ignore_index, grad_scale):
    """Drops the - eps / V term of the gradient."""
    x = np.asarray(logits, np.float64)
    y = np.asarray(targets, np.int64).reshape(-1)
    eps = float(np.float32(smoothing))
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    g = np.exp(x - lse[:, None])
    ignored = y == ignore_index
    bad = ~ignored & ((y < 0) | (y >= x.shape[1]))
    rows = np.nonzero(~ignored & ~bad)[0]
    g[rows, y[rows]] -= 1.0 - eps
    g[ignored] = 0.0
    g[bad] = np.nan
    return (float(np.float32(grad_scale)) * g).astype(np.float16)


# ------------------------------------------------- which pins must notice --

def _cases():
    fd = [(pins.test_ln_bwd_finite_differences, (3, 8)), (pins.test_ln_bwd_torch_autograd_and_invariants, ())]
    ln_fwd = [(pins.test_ln_constant_row_gives_beta, ()), (pins.test_ln_plus_minus_row_closed_form, ()),
              (pins.test_ln_matches_torch_and_one_pass, ())]
    sm = [(pins.test_softmax_matches_scipy_dense, ()), (pins.test_softmax_masked_scipy_and_zeros, ()),
          (pins.test_softmax_online_recurrence_agrees, ()), (pins.test_softmax_shift_invariance, ())]
    bdr = [(pins.test_bdr_p0_is_rounded_sum, ()), (pins.test_bdr_exposes_mask, ()), (pins.test_dropout_all_dropped, ())]
    emb = [(pins.test_embedding_fwd_exact_gather, ()), (pins.test_embedding_fwd_invalid_id_is_nan_row, ())]
    adam = [(pins.test_adam_step1_closed_form, ()), (pins.test_adam_zero_grad_is_pure_decay, ()),
            (pins.test_adam_matches_torch_optim, (True,)), (pins.test_adam_matches_torch_optim, (False,))]
    return [
        ("bias_dropout_residual", bdr_unscaled, bdr),
        ("bias_dropout_residual", bdr_bias_after_dropout, bdr),
        ("bias_relu_dropout", brd_relu_before_bias, [(pins.test_brd_p0_and_zeros, ()), (pins.test_dropout_all_dropped, ())]),
        ("layernorm_fwd", ln_fwd_unbiased, ln_fwd),
        ("layernorm_fwd", ln_fwd_eps_outside, ln_fwd),
        ("layernorm_bwd", ln_bwd_no_mean_term, fd),
        ("layernorm_bwd", ln_bwd_sign, fd),
        ("layernorm_bwd", ln_bwd_dgamma_raw_x, fd),
        ("layernorm_bwd", ln_bwd_dbeta_gamma, fd),
        ("softmax_fwd", softmax_mask_queries, sm),
        ("softmax_fwd", softmax_causal_strict, sm),
        ("softmax_bwd", softmax_bwd_no_dot, [(pins.test_softmax_bwd_finite_differences_and_invariants, ())]),
        ("softmax_bwd", softmax_bwd_dy_for_y, [(pins.test_softmax_bwd_finite_differences_and_invariants, ())]),
        ("embedding_fwd", emb_fwd_scale_on_position, emb),
        ("embedding_fwd", emb_fwd_position_is_batch, emb),
        ("embedding_bwd", emb_bwd_no_mask, [(pins.test_embedding_bwd_torch_autograd_and_conservation, ()),
                                            (pins.test_embedding_bwd_single_occurrence_and_accumulate, ())]),
        ("adam_workspace_step", adam_no_bias_correction, adam),
        ("adam_workspace_step", adam_eps_inside, adam),
        ("bias_dropout_residual_bwd", bdr_bwd_no_mask, [(pins.test_bdr_bwd_torch_autograd_and_special_cases, ())]),
        ("bias_relu_dropout_bwd", brd_bwd_gate_on_x, [(pins.test_brd_bwd_torch_autograd_and_output_gate, ())]),
        ("bias_qkv_split", qkv_split_heads_positions_swapped, [(pins.test_qkv_split_brute_force, ()),
                                                                (pins.test_qkv_split_inverse_and_autograd, ())]),
        ("cross_entropy_fwd", xent_spread_over_v_minus_1, [(pins.test_xent_matches_torch_and_logsumexp, (0.1,)),
                                                            (pins.test_xent_invariants_and_bad_targets, ())]),
        ("cross_entropy_bwd", xent_bwd_no_smoothing_floor, [(pins.test_xent_matches_torch_and_logsumexp, (0.1,)),
                                                             (pins.test_xent_invariants_and_bad_targets, ())]),
        ("bias_dropout_residual_layernorm", fused_ln_of_unrounded_sum,
         [(pins.test_bias_dropout_residual_layernorm_against_torch, (0.1,))]),
        ("bias_dropout_residual_layernorm", fused_ln_without_residual,
         [(pins.test_bias_dropout_residual_layernorm_against_torch, (0.0,))]),
        ("beam_candidates", beam_candidates_sign_flipped, [(golden.test_beam_candidates_hand_computed, ()),
                                                           (pins.test_hars_equals_full_sort, (3, 4, 50, 4))]),
        ("beam_candidates", beam_candidates_unrounded, [(golden.test_beam_candidates_hand_computed, ())]),
        ("hars_topk", hars_strict_threshold, [(pins.test_hars_worked_example_keeps_5_of_16, ()),
                                              (golden.test_hars_worked_example_counts, ())]),
    ]


@pytest.mark.parametrize("name,mutant,checks", _cases(), ids=lambda v: getattr(v, "__name__", None))
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, checks):
    monkeypatch.setattr(oracle, name, mutant)
    monkeypatch.setattr(oracle.ops, name, mutant)      # the oracle's own calls see it too
    failed = []
    for check, args in checks:
        try:
            check(*args)
        except Exception as e:      # an assertion, or a pin that cannot even run against the mistake
            failed.append(f"{check.__name__}: {type(e).__name__}")
    assert failed, f"no pin of oracle.{name} notices {mutant.__name__}: {mutant.__doc__}"


def test_pins_pass_on_the_oracle_itself():
    """The same checks, on the unmodified oracle, all pass (so a failure
    above is the planted mistake's doing)."""
    seen = set()
    for _, _, checks in _cases():
        for check, args in checks:
            if (check, args) not in seen:
                seen.add((check, args))
                check(*args)


# ------------------------------------------------ the dropout generator --

import test_oracle_philox as philox_pins  # noqa: E402
from oracle import philox  # noqa: E402
from test_oracle_philox import rocrand_ref  # noqa: E402,F401  (the host build of rocRAND's engine, a fixture)

_philox4x32 = philox.philox4x32


def philox_nine_rounds(counter, key, rounds=10):
    """Runs nine rounds instead of ten."""
    return _philox4x32(counter, key, rounds - 1)


def philox_swapped_multipliers(counter, key, rounds=10):
    """Multiplies c0 by M1 and c2 by M0 (the round constants exchanged)."""
    m = philox.MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(*(np.asarray(c, np.uint64) & m for c in counter))
    k0, k1 = np.uint64(key[0] & 0xFFFFFFFF), np.uint64(key[1] & 0xFFFFFFFF)
    for r in range(rounds):
        if r > 0:
            k0, k1 = (k0 + philox.PHILOX_W0) & m, (k1 + philox.PHILOX_W1) & m
        p0, p1 = philox.PHILOX_M1 * c0, philox.PHILOX_M0 * c2
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & m, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & m
    return c0, c1, c2, c3


def philox_key_bumped_first(counter, key, rounds=10):
    """Bumps the key before the first round as well."""
    k = ((key[0] + 0x9E3779B9) & 0xFFFFFFFF, (key[1] + 0xBB67AE85) & 0xFFFFFFFF)
    return _philox4x32(counter, k, rounds)


@pytest.mark.parametrize("mutant", [philox_nine_rounds, philox_swapped_multipliers, philox_key_bumped_first],
                         ids=lambda f: f.__name__)
def test_philox_pins_catch_planted_mistake(monkeypatch, rocrand_ref, mutant):  # noqa: F811
    monkeypatch.setattr(philox, "philox4x32", mutant)
    with pytest.raises(AssertionError):
        philox_pins.test_philox_matches_rocrand_engine(rocrand_ref, 0x0123456789ABCDEF, 3, 0)
