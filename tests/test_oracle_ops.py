"""Pins for the oracle's operator definitions (CPU only).

Each check is independent of the oracle's own code: closed forms, library
routines (torch / scipy on the CPU in float64), brute force, finite
differences, and invariants the mathematics fixes.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.ops import dropout_keep, dropout_scale

BITS = 16
SEED = 0x0123456789ABCDEF


def f16(a):
    return np.asarray(a, dtype=np.float16)


# ----------------------------------------------------------------------------
# bias + dropout + residual, bias + ReLU + dropout
# ----------------------------------------------------------------------------

def test_bdr_p0_is_rounded_sum():
    g = np.random.default_rng(1)
    x, r = f16(g.normal(size=(37, 24))), f16(g.normal(size=(37, 24)))
    b = f16(g.normal(0, 0.02, size=24))
    out = oracle.bias_dropout_residual(x, b, r, 0.0, SEED, 0, BITS)
    ref = (x.astype(np.float64) + b.astype(np.float64) + r.astype(np.float64)).astype(np.float16)
    np.testing.assert_array_equal(out, ref)


def test_bdr_exposes_mask():
    """x = 1, b = 0, r = 0: out is the scale where kept and 0 where dropped, in
    flat row-major order (checks that bias broadcasts over rows, the residual is
    added outside the dropout, and the element index is row * cols + col)."""
    rows, cols = 16, 40
    x = np.ones((rows, cols), np.float16)
    out = oracle.bias_dropout_residual(x, np.zeros(cols, np.float16), np.zeros_like(x), 0.3, SEED, 5, BITS)
    keep = dropout_keep(rows * cols, 0.3, SEED, 5, BITS).reshape(rows, cols)
    scale = 1.0 / (1.0 - np.floor(np.float64(np.float32(0.3)) * 65536) / 65536)
    np.testing.assert_array_equal(out, np.where(keep, scale, 0.0).astype(np.float16))
    # residual survives where the branch is dropped
    r = np.full((rows, cols), 2.0, np.float16)
    out2 = oracle.bias_dropout_residual(x, np.zeros(cols, np.float16), r, 0.3, SEED, 5, BITS)
    assert (out2[~keep] == 2.0).all()
    # bias is added before the dropout scale
    b = np.full(cols, 1.0, np.float16)
    out3 = oracle.bias_dropout_residual(x, b, np.zeros_like(x), 0.3, SEED, 5, BITS)
    np.testing.assert_array_equal(out3, np.where(keep, 2 * scale, 0.0).astype(np.float16))


def test_brd_p0_and_zeros():
    g = np.random.default_rng(2)
    x = f16(g.normal(size=(33, 48)))
    b = f16(g.normal(0, 0.5, size=48))
    out = oracle.bias_relu_dropout(x, b, 0.0, SEED, 1, BITS)
    ref = np.maximum(x.astype(np.float64) + b.astype(np.float64), 0).astype(np.float16)
    np.testing.assert_array_equal(out, ref)
    out = oracle.bias_relu_dropout(x, b, 0.25, SEED, 1, BITS)
    keep = dropout_keep(x.size, 0.25, SEED, 1, BITS).reshape(x.shape)
    pre = x.astype(np.float64) + b.astype(np.float64)
    assert (out[~keep] == 0).all() and (out[pre <= 0] == 0).all()
    sel = keep & (pre > 0)
    np.testing.assert_allclose(out[sel].astype(np.float64), pre[sel] / (1 - 16384 / 65536), rtol=1e-3)


def test_dropout_all_dropped():
    x = np.ones((4, 8), np.float16)
    out = oracle.bias_relu_dropout(x, np.zeros(8, np.float16), 1.0, SEED, 0, BITS)
    assert (out == 0).all()
    out = oracle.bias_dropout_residual(x, np.zeros(8, np.float16), x, 1.0, SEED, 0, BITS)
    assert (out == 1).all()


def test_bdr_bwd_torch_autograd_and_special_cases():
    """Autograd of residual + m * (x + b) in float64 gives d_x, d_bias and
    d_residual = dy; p = 0 passes dy through; p = 1 gives zeros; the backward's
    mask is the forward's (same flat index)."""
    g = np.random.default_rng(21)
    rows, cols, p, off = 29, 40, 0.5, 4      # scale 2: every float64 sum below is exact
    x, r, dy = (f16(g.normal(size=(rows, cols))) for _ in range(3))
    b = f16(g.normal(0, 0.02, size=cols))
    keep = dropout_keep(rows * cols, p, SEED, off, BITS).reshape(rows, cols)
    m = torch.tensor(keep * dropout_scale(p, BITS))
    xt, bt, rt = (torch.tensor(a.astype(np.float64), requires_grad=True) for a in (x, b, r))
    (rt + m * (xt + bt)).backward(torch.tensor(dy.astype(np.float64)))
    dx, db = oracle.bias_dropout_residual_bwd(dy, p, SEED, off, BITS)
    np.testing.assert_array_equal(dx, xt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(db, bt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(rt.grad.numpy(), dy.astype(np.float64))
    dx0, db0 = oracle.bias_dropout_residual_bwd(dy, 0.0, SEED, off, BITS)
    np.testing.assert_array_equal(dx0, dy)
    np.testing.assert_array_equal(db0, dy.astype(np.float64).sum(0).astype(np.float16))
    dx1, db1 = oracle.bias_dropout_residual_bwd(dy, 1.0, SEED, off, BITS)
    assert (dx1 == 0).all() and (db1 == 0).all()
    ones = np.ones((rows, cols), np.float16)
    fwd = oracle.bias_dropout_residual(ones, np.zeros(cols, np.float16), np.zeros_like(ones), p, SEED, off, BITS)
    np.testing.assert_array_equal(oracle.bias_dropout_residual_bwd(ones, p, SEED, off, BITS)[0], fwd)


def test_brd_bwd_torch_autograd_and_output_gate():
    """Autograd of m * relu(x + b) in float64; the gate [x + b > 0] * keep equals
    [forward output > 0] for fp16 inputs, including x + b = 0 and the smallest
    positive fp16 subnormal."""
    g = np.random.default_rng(22)
    rows, cols, p, off = 31, 48, 0.5, 1      # scale 2: every float64 sum below is exact
    x = f16(g.normal(size=(rows, cols)))
    b = f16(g.normal(0, 0.5, size=cols))
    b[:4] = 0
    x[:, 0] = 0                                        # pre = 0: ReLU's derivative 0
    x[:, 1] = np.float16(2.0 ** -24)                   # smallest positive pre
    x[:, 2] = -b[2]
    x[:, 5] = -b[5]                                    # pre = 0 with b != 0
    dy = f16(g.normal(size=(rows, cols)))
    keep = dropout_keep(rows * cols, p, SEED, off, BITS).reshape(rows, cols)
    m = torch.tensor(keep * dropout_scale(p, BITS))
    xt, bt = (torch.tensor(a.astype(np.float64), requires_grad=True) for a in (x, b))
    (m * torch.relu(xt + bt)).backward(torch.tensor(dy.astype(np.float64)))
    dx, db = oracle.bias_relu_dropout_bwd(dy, x, b, p, SEED, off, BITS)
    np.testing.assert_array_equal(dx, xt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(db, bt.grad.numpy().astype(np.float16))
    out = oracle.bias_relu_dropout(x, b, p, SEED, off, BITS)
    gate = (out.astype(np.float64) > 0) * dropout_scale(p, BITS)
    np.testing.assert_array_equal(dx, (dy.astype(np.float64) * gate).astype(np.float16))
    assert (out[:, 1] > 0).any() and (dx[:, 0] == 0).all() and (dx[:, 5] == 0).all()
    dx0, _ = oracle.bias_relu_dropout_bwd(dy, x, b, 0.0, SEED, off, BITS)
    pre = x.astype(np.float64) + b.astype(np.float64)
    np.testing.assert_array_equal(dx0, np.where(pre > 0, dy, np.float16(0)))


def test_ew_bwd_inexact_scale_within_one_ulp():
    """With p = 0.25 (scale 4/3, inexact in binary) d_x is still exact per
    element, and d_bias can sit on an fp16 rounding tie whose side depends on
    float64 summation order: it agrees with autograd to one fp16 ulp."""
    g = np.random.default_rng(23)
    rows, cols, p, off = 31, 48, 0.25, 1
    x, dy = f16(g.normal(size=(rows, cols))), f16(g.normal(size=(rows, cols)))
    b = f16(g.normal(0, 0.5, size=cols))
    keep = dropout_keep(rows * cols, p, SEED, off, BITS).reshape(rows, cols)
    m = torch.tensor(keep * dropout_scale(p, BITS))
    for relu in (False, True):
        xt, bt = (torch.tensor(a.astype(np.float64), requires_grad=True) for a in (x, b))
        y = m * (torch.relu(xt + bt) if relu else (xt + bt))
        y.backward(torch.tensor(dy.astype(np.float64)))
        dx, db = (oracle.bias_relu_dropout_bwd(dy, x, b, p, SEED, off, BITS) if relu
                  else oracle.bias_dropout_residual_bwd(dy, p, SEED, off, BITS))
        np.testing.assert_array_equal(dx, xt.grad.numpy().astype(np.float16))
        ref = bt.grad.numpy()
        np.testing.assert_allclose(db.astype(np.float64), ref, rtol=2.0 ** -10, atol=2.0 ** -24)


# ----------------------------------------------------------------------------
# Bias + Q/K/V head split
# ----------------------------------------------------------------------------

def test_qkv_split_brute_force():
    """Every output element against its defining index formula, loop by loop."""
    g = np.random.default_rng(31)
    batch, seq, heads, d = 2, 3, 2, 4
    H = heads * d
    qkv = f16(g.normal(size=(batch * seq, 3 * H)))
    bias = f16(g.normal(size=3 * H))
    out = oracle.bias_qkv_split(qkv, bias, batch, seq, heads)
    assert out.shape == (3, batch, heads, seq, d)
    for k in range(3):
        for b in range(batch):
            for h in range(heads):
                for l in range(seq):
                    for j in range(d):
                        c = k * H + h * d + j
                        want = np.float16(float(qkv[b * seq + l, c]) + float(bias[c]))
                        assert out[k, b, h, l, j] == want
    dout = f16(g.normal(size=out.shape))
    dq, db = oracle.bias_qkv_split_bwd(dout, batch, seq, heads)
    for k in range(3):
        for b in range(batch):
            for h in range(heads):
                for l in range(seq):
                    for j in range(d):
                        assert dq[b * seq + l, k * H + h * d + j] == dout[k, b, h, l, j]
    for c in range(3 * H):
        k, h, j = c // H, (c % H) // d, c % d
        assert db[c] == np.float16(sum(float(dout[k, b, h, l, j]) for b in range(batch) for l in range(seq)))


def test_qkv_split_inverse_and_autograd():
    g = np.random.default_rng(32)
    batch, seq, heads, d = 3, 5, 4, 8
    H = heads * d
    qkv = f16(g.normal(size=(batch * seq, 3 * H)))
    out = oracle.bias_qkv_split(qkv, np.zeros(3 * H, np.float16), batch, seq, heads)
    np.testing.assert_array_equal(oracle.bias_qkv_split_bwd(out, batch, seq, heads)[0], qkv)
    bias = f16(g.normal(size=3 * H))
    xt = torch.tensor(qkv.astype(np.float64), requires_grad=True)
    bt = torch.tensor(bias.astype(np.float64), requires_grad=True)
    y = (xt + bt).view(batch, seq, 3, heads, d).permute(2, 0, 3, 1, 4)
    dout = f16(g.normal(size=(3, batch, heads, seq, d)))
    y.backward(torch.tensor(dout.astype(np.float64)))
    dq, db = oracle.bias_qkv_split_bwd(dout, batch, seq, heads)
    np.testing.assert_array_equal(dq, xt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(db, bt.grad.numpy().astype(np.float16))


# ----------------------------------------------------------------------------
# Cross-entropy criterion
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [0.0, 0.1, 1.0])
def test_xent_matches_torch_and_logsumexp(eps):
    g = np.random.default_rng(41)
    rows, v, ignore = 23, 57, 3
    x = f16(g.normal(0, 3, size=(rows, v)))
    y = g.integers(0, v, size=rows).astype(np.int32)
    y[[2, 7]] = ignore
    loss, lse = oracle.cross_entropy_fwd(x, y, eps, ignore)
    x64 = torch.tensor(x.astype(np.float64), requires_grad=True)
    ref = torch.nn.functional.cross_entropy(x64, torch.tensor(y.astype(np.int64)), reduction="none",
                                            label_smoothing=eps, ignore_index=ignore)
    np.testing.assert_array_equal(loss, ref.detach().numpy().astype(np.float32))
    np.testing.assert_array_equal(lse, scipy.special.logsumexp(x.astype(np.float64), axis=1).astype(np.float32))
    assert loss[2] == 0 and loss[7] == 0
    (0.75 * ref).sum().backward()
    dx = oracle.cross_entropy_bwd(x, y, eps, ignore, 0.75)
    np.testing.assert_array_equal(dx, x64.grad.numpy().astype(np.float16))
    assert (dx[[2, 7]] == 0).all()


def test_xent_invariants_and_bad_targets():
    """Each gradient row sums to 0 (softmax and the smoothed one-hot both sum
    to 1); a uniform row has loss log V; a target outside [0, V) gives NaN."""
    g = np.random.default_rng(42)
    x = f16(g.normal(size=(9, 40)))
    y = g.integers(0, 40, size=9).astype(np.int32)
    y[4] = 40
    y[5] = -7
    loss, _ = oracle.cross_entropy_fwd(x, y, 0.1, -1)
    assert np.isnan(loss[4]) and np.isnan(loss[5]) and np.isfinite(np.delete(loss, [4, 5])).all()
    dx = oracle.cross_entropy_bwd(x, y, 0.1, -1, 1.0)
    assert np.isnan(dx[4]).all() and np.isnan(dx[5]).all()
    x64 = x.astype(np.float64)
    lse = scipy.special.logsumexp(x64, axis=1, keepdims=True)
    full = np.exp(x64 - lse) - 0.1 / 40
    full[np.arange(9), np.clip(y, 0, 39)] -= 0.9
    np.testing.assert_allclose(np.delete(full, [4, 5], axis=0).sum(1), 0, atol=1e-12)
    u, _ = oracle.cross_entropy_fwd(np.zeros((2, 1000), np.float16), np.array([0, 999], np.int32), 0.3, -1)
    np.testing.assert_allclose(u, np.log(1000), rtol=1e-7)


# ----------------------------------------------------------------------------
# HARS beam-search top-k
# ----------------------------------------------------------------------------

def _full_sort_topk(lp, bs, k):
    """Every candidate sorted: value descending (NaN first, -0 below +0), then
    index.  The candidates come from torch's float32 addition, not from the
    oracle."""
    c = torch.from_numpy(np.ascontiguousarray(lp, np.float32))
    if bs is not None:
        c = c + torch.from_numpy(np.ascontiguousarray(bs, np.float32))[:, :, None]
    c = c.numpy()
    batch = c.shape[0]
    flat = c.reshape(batch, -1)
    out_s, out_i = [], []
    for b in range(batch):
        vals = flat[b].astype(np.float64)
        nan = np.isnan(vals)
        neg0 = (vals == 0) & np.signbit(vals)
        order = sorted(range(vals.size), key=lambda j: (0 if nan[j] else 1, -vals[j] if not nan[j] else 0,
                                                       1 if neg0[j] else 0, j))
        best = np.array(order[:k])
        out_i.append(best)
        out_s.append(flat[b][best])
    return np.array(out_s, np.float32), np.array(out_i, np.int32)


@pytest.mark.parametrize("batch,beam,v,k", [(3, 4, 50, 4), (2, 1, 9, 9), (2, 3, 2, 4), (1, 5, 40, 1)])
def test_hars_equals_full_sort(batch, beam, v, k):
    g = np.random.default_rng(batch * 100 + v)
    lp = g.normal(size=(batch, beam, v)).astype(np.float32)
    bs = g.normal(size=(batch, beam)).astype(np.float32)
    if v > 3:
        lp[0, 0, :3] = lp[0, 0, 3]            # ties: the smaller index ranks first
    s, i, surv = oracle.hars_topk(lp, bs, k, return_survivors=True)
    s2, i2 = _full_sort_topk(lp, bs, k)
    np.testing.assert_array_equal(i, i2)
    np.testing.assert_array_equal(s.view(np.uint32), s2.view(np.uint32))
    assert (surv >= k).all() and (surv <= beam * v).all()


def test_hars_special_values_and_ties():
    lp = np.zeros((1, 2, 6), np.float32)
    lp[0, 0, 1] = -0.0
    lp[0, 1, 4] = np.nan
    lp[0, 1, 5] = np.inf
    s, i = oracle.hars_topk(lp, None, 4)
    s2, i2 = _full_sort_topk(lp, None, 4)
    np.testing.assert_array_equal(i, i2)
    assert i[0, 0] == 10 and i[0, 1] == 11            # NaN first, then +inf
    assert list(i[0, 2:]) == [0, 2]                   # +0 ties by index; the -0 at 1 ranks below them
    s, i = oracle.hars_topk(np.ones((1, 3, 4), np.float32), None, 5)
    assert list(i[0]) == [0, 1, 2, 3, 4]


def test_hars_worked_example_keeps_5_of_16():
    """Beam 2, vocabulary 8, k = 2: 16 candidates, 5 of them at or above the
    threshold (groups of 4: beam 0 maxima 10 and 8.75, beam 1 maxima 9.5 and
    8.5, so R = max(8.75, 8.5))."""
    lp = np.array([[[10, 1, 9, 2, 3, 8.75, 4, 7], [9.5, 9.25, 0, 0, 8.5, 0, 0, 0]]], np.float32)
    s, i, surv = oracle.hars_topk(lp, None, 2, return_survivors=True)
    assert lp.size == 16 and surv[0] == 5
    assert list(i[0]) == [0, 8] and list(s[0]) == [10.0, 9.5]


# ----------------------------------------------------------------------------
# LayerNorm
# ----------------------------------------------------------------------------

def test_ln_constant_row_gives_beta():
    h = 64
    x = np.full((3, h), 1.5, np.float16)
    g = np.random.default_rng(3)
    gamma, beta = f16(g.uniform(0.5, 1.5, h)), f16(g.normal(0, 0.1, h))
    y, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, 1e-5)
    np.testing.assert_array_equal(y, np.broadcast_to(beta, y.shape))
    assert (mean == np.float32(1.5)).all()
    np.testing.assert_allclose(rstd, 1 / np.sqrt(np.float64(np.float32(1e-5))), rtol=1e-7)


def test_ln_plus_minus_row_closed_form():
    """Row (a, -a, a, -a, ...): mean 0, var a^2, y = +-a/sqrt(a^2 + eps)."""
    a, h, eps = 0.75, 32, 1e-5
    x = f16(np.tile([a, -a], h // 2)[None, :])
    gamma = np.ones(h, np.float16)
    beta = np.zeros(h, np.float16)
    y, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, eps)
    expect = np.tile([a, -a], h // 2) / np.sqrt(a * a + np.float64(np.float32(eps)))
    np.testing.assert_array_equal(y[0], expect.astype(np.float16))
    assert mean[0] == 0.0


def test_ln_matches_torch_and_one_pass():
    g = np.random.default_rng(4)
    x = f16(g.normal(0.3, 1.7, size=(50, 96)))
    gamma, beta = f16(g.uniform(0.5, 1.5, 96)), f16(g.normal(0, 0.1, 96))
    eps = 1e-5
    y, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, eps)
    xt = torch.tensor(x.astype(np.float64))
    ref = torch.nn.functional.layer_norm(xt, (96,), torch.tensor(gamma.astype(np.float64)),
                                         torch.tensor(beta.astype(np.float64)), float(np.float32(eps)))
    np.testing.assert_array_equal(y, ref.numpy().astype(np.float16))
    # one-pass statistics (E[x^2] - E[x]^2) agree with the two-pass ones in fp64
    x64 = x.astype(np.float64)
    mu1 = x64.mean(1)
    var1 = (x64 * x64).mean(1) - mu1 * mu1
    np.testing.assert_allclose(1 / np.sqrt(var1 + np.float64(np.float32(eps))), rstd, rtol=1e-6)
    np.testing.assert_allclose(mu1, mean, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("p", [0.0, 0.1])
def test_bias_dropout_residual_layernorm_against_torch(p):
    """The fused sub-layer output block: torch float64 for the sum (rounded to
    fp16, the stored z) and for layer_norm; the mask from the Philox keep
    function (pinned against rocRAND's engine) and the page-derived scale."""
    g = np.random.default_rng(12)
    rows, h, seed, off = 40, 96, 0x1234, 2
    x, r = f16(g.normal(size=(rows, h))), f16(g.normal(size=(rows, h)))
    b, gamma, beta = f16(g.normal(0, 0.02, h)), f16(g.uniform(0.5, 1.5, h)), f16(g.normal(0, 0.1, h))
    eps = 1e-5
    z, y, mean, rstd = oracle.bias_dropout_residual_layernorm(x, b, r, gamma, beta, p, seed, off, 16, eps)
    keep = dropout_keep(np.arange(rows * h, dtype=np.uint64), p, seed, off, 16).reshape(rows, h)
    t = lambda a: torch.tensor(np.asarray(a, np.float64))  # noqa: E731
    zt = t(r) + t(keep) * dropout_scale(p, 16) * (t(x) + t(b))
    z_ref = zt.numpy().astype(np.float16)
    np.testing.assert_array_equal(z, z_ref)
    z64 = t(z_ref)
    y_ref = torch.nn.functional.layer_norm(z64, (h,), t(gamma), t(beta), float(np.float32(eps)))
    np.testing.assert_array_equal(y, y_ref.numpy().astype(np.float16))
    var, mu = torch.var_mean(z64, dim=1, unbiased=False)
    np.testing.assert_allclose(mean, mu.numpy(), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(rstd, (1 / torch.sqrt(var + float(np.float32(eps)))).numpy(), rtol=1e-7)
    # a constant residual row with x + bias = 0 everywhere normalises to beta
    z, y, _, _ = oracle.bias_dropout_residual_layernorm(np.zeros((2, h), np.float16), np.zeros(h, np.float16),
                                                        np.full((2, h), 3.0, np.float16), gamma, beta, p, seed, off,
                                                        16, eps)
    assert np.all(z == np.float16(3.0)) and np.array_equal(y, np.broadcast_to(beta, y.shape))


def _ln_fwd64(x, gamma, beta, eps):
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


@pytest.mark.parametrize("rows,h", [(3, 8), (2, 16)])
def test_ln_bwd_finite_differences(rows, h):
    """Central differences of sum(dy * LN(x)) in fp64 (h = 1e-6)."""
    g = np.random.default_rng(5 + h)
    x = f16(g.normal(size=(rows, h)))
    dy = f16(g.normal(size=(rows, h)))
    gamma, beta = f16(g.uniform(0.5, 1.5, h)), f16(g.normal(0, 0.1, h))
    eps = float(np.float32(1e-5))
    x64, dy64, g64, b64 = (a.astype(np.float64) for a in (x, dy, gamma, beta))
    mu = x64.mean(-1)
    rstd = 1 / np.sqrt(((x64 - mu[:, None]) ** 2).mean(-1) + eps)
    dx, dgamma, dbeta = oracle.layernorm_bwd(dy, x, gamma, mu, rstd)

    def loss(xx, gg, bb):
        return (dy64 * _ln_fwd64(xx, gg, bb, eps)).sum()
    step = 1e-6
    num_dx = np.zeros_like(x64)
    for i in range(rows):
        for j in range(h):
            e = np.zeros_like(x64)
            e[i, j] = step
            num_dx[i, j] = (loss(x64 + e, g64, b64) - loss(x64 - e, g64, b64)) / (2 * step)
    num_dg = np.array([(loss(x64, g64 + step * np.eye(h)[j], b64) - loss(x64, g64 - step * np.eye(h)[j], b64))
                       / (2 * step) for j in range(h)])
    num_db = np.array([(loss(x64, g64, b64 + step * np.eye(h)[j]) - loss(x64, g64, b64 - step * np.eye(h)[j]))
                       / (2 * step) for j in range(h)])
    np.testing.assert_allclose(dx.astype(np.float64), num_dx, rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(dgamma.astype(np.float64), num_dg, rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(dbeta.astype(np.float64), num_db, rtol=2e-3, atol=2e-3)


def test_ln_bwd_torch_autograd_and_invariants():
    g = np.random.default_rng(6)
    rows, h = 40, 64
    x = f16(g.normal(size=(rows, h)))
    dy = f16(g.normal(size=(rows, h)))
    gamma, beta = f16(g.uniform(0.5, 1.5, h)), f16(g.normal(0, 0.1, h))
    eps = float(np.float32(1e-5))
    xt = torch.tensor(x.astype(np.float64), requires_grad=True)
    gt = torch.tensor(gamma.astype(np.float64), requires_grad=True)
    bt = torch.tensor(beta.astype(np.float64), requires_grad=True)
    y = torch.nn.functional.layer_norm(xt, (h,), gt, bt, eps)
    y.backward(torch.tensor(dy.astype(np.float64)))
    x64 = x.astype(np.float64)
    mu = x64.mean(-1)
    rstd = 1 / np.sqrt(((x64 - mu[:, None]) ** 2).mean(-1) + eps)
    dx, dgamma, dbeta = oracle.layernorm_bwd(dy, x, gamma, mu, rstd)
    np.testing.assert_array_equal(dx, xt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(dgamma, gt.grad.numpy().astype(np.float16))
    np.testing.assert_array_equal(dbeta, bt.grad.numpy().astype(np.float16))
    # invariants of the exact gradient; sum(dx * xhat) = 0 needs eps = 0
    rstd0 = 1 / np.sqrt(((x64 - mu[:, None]) ** 2).mean(-1))
    dx0 = oracle.layernorm_bwd(dy, x, gamma, mu, rstd0)[0]
    xhat = (x64 - mu[:, None]) * rstd0[:, None]
    gd = gamma.astype(np.float64) * dy.astype(np.float64)
    dx64 = rstd0[:, None] * (gd - gd.mean(-1, keepdims=True) - xhat * (gd * xhat).mean(-1, keepdims=True))
    np.testing.assert_array_equal(dx0, dx64.astype(np.float16))
    np.testing.assert_allclose(dx64.sum(-1), 0, atol=1e-10)
    np.testing.assert_allclose((dx64 * xhat).sum(-1), 0, atol=1e-10)
    np.testing.assert_array_equal(dbeta, dy.astype(np.float64).sum(0).astype(np.float16))


# ----------------------------------------------------------------------------
# Softmax
# ----------------------------------------------------------------------------

def test_softmax_matches_scipy_dense():
    g = np.random.default_rng(7)
    x = f16(g.normal(0, 3, size=(2, 3, 5, 40)))
    y = oracle.softmax_fwd(x)
    ref = scipy.special.softmax(x.astype(np.float64), axis=-1)
    np.testing.assert_array_equal(y, ref.astype(np.float16))
    # rows sum to 1 within fp16 rounding of each entry
    s = y.astype(np.float64).sum(-1)
    assert np.all(np.abs(s - 1) <= 40 * 2.0 ** -11 + 1e-12)


def test_softmax_masked_scipy_and_zeros():
    g = np.random.default_rng(8)
    b, h, q, k = 3, 2, 6, 24
    x = f16(g.normal(0, 3, size=(b, h, q, k)))
    lens = np.array([24, 5, 0], np.int32)
    y = oracle.softmax_fwd(x, lens, causal=True)
    for bi in range(b):
        for hi in range(h):
            for qi in range(q):
                n = min(int(lens[bi]), qi + 1)
                row = y[bi, hi, qi]
                assert (row[n:] == 0).all()
                if n:
                    ref = scipy.special.softmax(x[bi, hi, qi, :n].astype(np.float64))
                    np.testing.assert_array_equal(row[:n], ref.astype(np.float16))
    assert (y[2] == 0).all()                                  # no valid key at all
    # constant row: 1/|valid| ; shift invariance
    c = np.zeros((1, 1, 1, 24), np.float16)
    np.testing.assert_array_equal(oracle.softmax_fwd(c, np.array([7], np.int32))[0, 0, 0, :7],
                                  np.float16(1 / 7))


def test_softmax_online_recurrence_agrees():
    """Block-wise running max m and normaliser l (online softmax) reach the
    same normaliser as the two-pass form; the oracle's rows equal exp(x-m)/l."""
    g = np.random.default_rng(9)
    x = g.normal(0, 3, size=(20, 256)).astype(np.float16).astype(np.float64)
    m = np.full(20, -np.inf)
    l = np.zeros(20)
    for blk in np.split(x, 8, axis=1):
        m_new = np.maximum(m, blk.max(1))
        l = l * np.exp(m - m_new) + np.exp(blk - m_new[:, None]).sum(1)
        m = m_new
    online = np.exp(x - m[:, None]) / l[:, None]
    y = oracle.softmax_fwd(f16(x)[None, None])[0, 0]
    np.testing.assert_array_equal(y, online.astype(np.float16))
    # argmax of the output equals argmax of the input (lowest index on ties)
    assert (np.argmax(x, 1) == np.argmax(y.astype(np.float64), 1)).mean() > 0.9


def test_softmax_shift_invariance():
    g = np.random.default_rng(10)
    x = g.integers(-20, 20, size=(1, 1, 4, 32)).astype(np.float16)   # exact under +8
    y1 = oracle.softmax_fwd(x)
    y2 = oracle.softmax_fwd(f16(x.astype(np.float64) + 8))
    np.testing.assert_array_equal(y1, y2)


def test_softmax_bwd_finite_differences_and_invariants():
    g = np.random.default_rng(11)
    k = 12
    x = g.normal(0, 1, size=(1, 1, 2, k))
    dy = g.normal(size=(2, k))
    y64 = scipy.special.softmax(x[0, 0], axis=-1)
    dx = oracle.softmax_bwd(y64, dy).astype(np.float64)
    num = np.zeros((2, k))
    h = 1e-6
    for i in range(2):
        for j in range(k):
            e = np.zeros(k)
            e[j] = h
            num[i, j] = ((scipy.special.softmax(x[0, 0, i] + e) * dy[i]).sum()
                         - (scipy.special.softmax(x[0, 0, i] - e) * dy[i]).sum()) / (2 * h)
    np.testing.assert_allclose(dx, num, rtol=2e-3, atol=1e-3)
    # torch autograd
    xt = torch.tensor(x[0, 0], requires_grad=True)
    torch.softmax(xt, -1).backward(torch.tensor(dy))
    np.testing.assert_array_equal(oracle.softmax_bwd(y64, dy), xt.grad.numpy().astype(np.float16))
    # constant dy -> 0 ; rows of the exact gradient sum to 0
    np.testing.assert_array_equal(oracle.softmax_bwd(y64, np.ones((2, k))), np.zeros((2, k), np.float16))
    exact = y64 * (dy - (y64 * dy).sum(-1, keepdims=True))
    np.testing.assert_allclose(exact.sum(-1), 0, atol=1e-12)


# ----------------------------------------------------------------------------
# Embedding
# ----------------------------------------------------------------------------

def test_embedding_fwd_exact_gather():
    """p = 0 and P = 0: out = s * E[ids], exact for a power-of-two scale."""
    g = np.random.default_rng(12)
    v, h, b, l = 50, 16, 3, 7
    E = f16(g.normal(0, 0.25, size=(v, h)))
    ids = g.integers(0, v, size=(b, l)).astype(np.int32)
    out = oracle.embedding_fwd(ids, E, np.zeros((l, h), np.float16), 32.0, 0.0, SEED, 3, BITS)
    np.testing.assert_array_equal(out, (E[ids.reshape(-1)].astype(np.float64) * 32).astype(np.float16))
    # against torch's embedding with positions and dropout applied by hand
    P = f16(g.normal(size=(l + 3, h)))
    out = oracle.embedding_fwd(ids, E, P, 32.0, 0.2, SEED, 3, BITS)
    emb = torch.nn.functional.embedding(torch.tensor(ids.reshape(-1).astype(np.int64)),
                                        torch.tensor(E.astype(np.float64))).numpy()
    pos = np.tile(np.arange(l), b)
    keep = dropout_keep(b * l * h, 0.2, SEED, 3, BITS).reshape(b * l, h)
    ref = (32 * emb + P[pos].astype(np.float64)) * keep * dropout_scale(0.2, BITS)
    np.testing.assert_array_equal(out, ref.astype(np.float16))


def test_embedding_fwd_invalid_id_is_nan_row():
    E = np.ones((4, 8), np.float16)
    ids = np.array([[0, 4, -1, 3]], np.int32)
    out = oracle.embedding_fwd(ids, E, np.zeros((4, 8), np.float16), 1.0, 0.0, SEED, 3, BITS)
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert (out[0] == 1).all() and (out[3] == 1).all()


def test_embedding_bwd_torch_autograd_and_conservation():
    g = np.random.default_rng(13)
    v, h, b, l = 40, 24, 4, 9
    ids = g.integers(0, 8, size=(b, l)).astype(np.int32)      # many repeats
    dy = f16(g.normal(size=(b * l, h)))
    s, p = 32.0, 0.1
    grad = oracle.embedding_bwd(ids, dy, v, s, p, SEED, 3, BITS)
    keep = dropout_keep(b * l * h, p, SEED, 3, BITS).reshape(b * l, h)
    m = keep * dropout_scale(p, BITS)
    Et = torch.zeros((v, h), dtype=torch.float64, requires_grad=True)
    out = s * torch.nn.functional.embedding(torch.tensor(ids.reshape(-1).astype(np.int64)), Et) * torch.tensor(m)
    out.backward(torch.tensor(dy.astype(np.float64)))
    np.testing.assert_array_equal(grad, Et.grad.numpy().astype(np.float32))
    # mass conservation and untouched rows
    contrib = s * m * dy.astype(np.float64)
    err = np.abs(grad.astype(np.float64).sum(0) - contrib.sum(0))
    assert np.all(err <= 1e-6 * np.abs(contrib).sum(0))        # fp32 rounding of each row only
    assert (grad[8:] == 0).all()


def test_embedding_bwd_single_occurrence_and_accumulate():
    dy = f16(np.arange(16).reshape(2, 8) / 8)
    ids = np.array([[3, 1]], np.int32)
    grad = oracle.embedding_bwd(ids, dy, 5, 32.0, 0.0, SEED, 3, BITS)
    np.testing.assert_array_equal(grad[3], (32 * dy[0].astype(np.float64)).astype(np.float32))
    np.testing.assert_array_equal(grad[1], (32 * dy[1].astype(np.float64)).astype(np.float32))
    acc = oracle.embedding_bwd(ids, dy, 5, 32.0, 0.0, SEED, 3, BITS, grad_in=grad)
    np.testing.assert_array_equal(acc, 2 * grad)
    bad = oracle.embedding_bwd(np.array([[7, -2]], np.int32), dy, 5, 32.0, 0.0, SEED, 3, BITS)
    assert (bad == 0).all()


# ----------------------------------------------------------------------------
# Adam
# ----------------------------------------------------------------------------

def test_adam_step1_closed_form():
    """At t = 1, m_hat = g and v_hat = g^2, so the step is lr*(g/(|g|+eps) + wd*p)."""
    g = np.random.default_rng(14)
    p = f16(g.normal(0, 0.02, 1000))
    gr = f16(g.normal(0, 1e-3, 1000))
    lr, wd, eps = 1e-4, 0.01, 1e-8
    p1, m1, v1 = oracle.adam_workspace_step(p, gr, np.zeros(1000, np.float32), np.zeros(1000, np.float32),
                                            lr, 0.9, 0.98, eps, wd, 1)
    p64, g64 = p.astype(np.float64), gr.astype(np.float64)
    lr64, wd64, eps64 = (float(np.float32(v)) for v in (lr, wd, eps))
    expect = p64 - lr64 * (g64 / (np.abs(g64) + eps64) + wd64 * p64)
    np.testing.assert_array_equal(p1, expect.astype(np.float16))
    np.testing.assert_allclose(m1, (1 - np.float64(np.float32(0.9))) * g64, rtol=1e-6)


def test_adam_zero_grad_is_pure_decay():
    p = f16(np.linspace(-2, 2, 64))
    z = np.zeros(64, np.float16)
    p1, m1, v1 = oracle.adam_workspace_step(p, z, np.zeros(64, np.float32), np.zeros(64, np.float32),
                                            0.5, 0.9, 0.98, 1e-8, 0.1, 1)
    lr, wd = float(np.float32(0.5)), float(np.float32(0.1))
    np.testing.assert_array_equal(p1, (p.astype(np.float64) * (1 - lr * wd)).astype(np.float16))
    assert (m1 == 0).all() and (v1 == 0).all()


@pytest.mark.parametrize("decoupled", [True, False])
def test_adam_matches_torch_optim(decoupled):
    """Ten steps against torch.optim.AdamW / Adam in fp64.  The oracle's fp16
    parameter storage is undone by feeding torch the same fp16-rounded
    parameter each step and comparing one step at a time."""
    g = np.random.default_rng(15)
    n = 512
    p = f16(g.normal(0, 0.02, n))
    gr = f16(g.normal(0, 1e-3, n))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hyper = dict(lr=1e-3, betas=(0.9, 0.98), eps=1e-8, weight_decay=0.01)
    f32 = lambda a: float(np.float32(a))  # noqa: E731
    t_hyper = dict(lr=f32(1e-3), betas=(f32(0.9), f32(0.98)), eps=f32(1e-8), weight_decay=f32(0.01))
    pt = torch.tensor(p.astype(np.float64), requires_grad=True)
    opt = (torch.optim.AdamW if decoupled else torch.optim.Adam)([pt], **t_hyper)
    for step in range(1, 11):
        with torch.no_grad():
            pt.copy_(torch.tensor(p.astype(np.float64)))
        pt.grad = torch.tensor(gr.astype(np.float64))
        opt.step()
        p, m, v = oracle.adam_workspace_step(p, gr, m, v, hyper["lr"], 0.9, 0.98, 1e-8, 0.01, step,
                                             decoupled_wd=decoupled)
        st = opt.state[pt]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-6, atol=1e-16)
        d = np.abs(p.astype(np.float64) - pt.detach().numpy())
        assert np.all(d <= np.spacing(np.abs(pt.detach().numpy()).astype(np.float16)).astype(np.float64))


def test_adam_grad_scale():
    p = f16(np.linspace(-1, 1, 32))
    gr = f16(np.linspace(-1, 1, 32) * 1e-3)
    z = np.zeros(32, np.float32)
    a = oracle.adam_workspace_step(p, gr, z, z, 1e-3, 0.9, 0.98, 1e-8, 0.0, 3, grad_scale=1.0)
    b = oracle.adam_workspace_step(p, f16(gr.astype(np.float64) * 512), z, z, 1e-3, 0.9, 0.98, 1e-8, 0.0, 3,
                                   grad_scale=512.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], rtol=1e-6)
