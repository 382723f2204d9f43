"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Bars (written here, not in the oracle):
* dropout masks, argmax and indexing: bit-exact;
* fp16 outputs: an element fails iff |a-b| > 2e-3 and |a-b| > 1e-2 |b|;
* fp32 statistics and moments: |a-b| <= 1e-5 * max(|b|, floor).
Shapes cover several tiles, ragged tails, the vector and element-wise paths,
the empty case and the workloads' full sizes.
"""
import re

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import fp16_mismatch
from golden_data import hars_example

pytestmark = pytest.mark.gpu

BITS = 16
SEED = synth.DROPOUT_SEED


@pytest.fixture(scope="module")
def ls():
    from non_gemm_amd import _lib, ops
    _lib.load()
    assert _lib.dropout_decision_bits() == BITS
    return ops


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_fp16(a, b, what):
    bad = fp16_mismatch(a, b)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} out of tolerance; first at {i}: "
                             f"{np.asarray(a)[i]} vs oracle {np.asarray(b)[i]}")


def assert_fp32(a, b, what, floor=1e-30):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    tol = 1e-5 * np.maximum(np.abs(b), floor)
    bad = ~(np.abs(a - b) <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} out of tolerance; first at {i}: "
                             f"{a[i]} vs oracle {b[i]}")


def last_dispatch():
    from non_gemm_amd import _lib
    return _lib.last_dispatch()


# ----------------------------------------------------------------------------
# Dropout mask
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n,p,seed,offset", [
    (1, 0.1, SEED, 0),
    (1_000_003, 0.1, SEED, 0),
    (65_541, 0.5, 7, 3),
    (4096 * 768, 0.1, SEED, 2),
    (12_345, 0.0, 1, 1),
    (12_345, 1.0, 1, 1),
    (999, 0.999, 2**64 - 1, 2**64 - 1),
])
def test_dropout_mask_bit_exact(ls, n, p, seed, offset):
    keep = host(ls.dropout_mask(n, p, seed, offset)).astype(bool)
    ref = oracle.dropout_keep(n, p, seed, offset, BITS)
    assert keep.shape == ref.shape
    assert np.array_equal(keep, ref), f"{int((keep != ref).sum())} decisions differ"


# ----------------------------------------------------------------------------
# bias + dropout + residual / bias + ReLU + dropout
# ----------------------------------------------------------------------------

EW_SHAPES = [(128, 256), (4096, 768), (8192, 1024), (37, 24), (5, 1000), (3, 13), (1, 8), (0, 64)]


@pytest.mark.parametrize("rows,cols", EW_SHAPES)
@pytest.mark.parametrize("p", [0.1, 0.0])
def test_bias_dropout_residual(ls, rows, cols, p):
    g = np.random.default_rng(rows * 1000 + cols)
    x = synth.normal16(g, (rows, cols), 1.0)
    r = synth.normal16(g, (rows, cols), 1.0)
    b = synth.normal16(g, (cols,), 0.02)
    out = host(ls.bias_dropout_residual(dev(x), dev(b), dev(r), p, SEED, synth.SITE_ATTN_OUT))
    ref = oracle.bias_dropout_residual(x, b, r, p, SEED, synth.SITE_ATTN_OUT, BITS)
    assert_fp16(out, ref, f"bias_dropout_residual {rows}x{cols} p={p} [{last_dispatch()}]")


@pytest.mark.parametrize("rows,cols", [(128, 256), (333, 40), (7, 13)])
def test_bias_dropout_residual_mask_exposed(ls, rows, cols):
    """x = 1, b = 0, r = 0: the output is exactly the mask times the scale."""
    x = np.ones((rows, cols), np.float16)
    z = np.zeros((rows, cols), np.float16)
    out = host(ls.bias_dropout_residual(dev(x), dev(np.zeros(cols, np.float16)), dev(z), 0.25, 11, 4))
    keep = oracle.dropout_keep(rows * cols, 0.25, 11, 4, BITS).reshape(rows, cols)
    assert np.array_equal(out != 0, keep)
    assert np.all(out[keep] == np.float16(1 / 0.75))


def test_bias_dropout_residual_aliasing_and_unaligned(ls):
    g = np.random.default_rng(5)
    rows, cols = 300, 64
    x = synth.normal16(g, (rows, cols), 1.0)
    r = synth.normal16(g, (rows, cols), 1.0)
    b = synth.normal16(g, (cols,), 0.02)
    ref = oracle.bias_dropout_residual(x, b, r, 0.1, SEED, 0, BITS)
    rt = dev(r)
    ls.bias_dropout_residual(dev(x), dev(b), rt, 0.1, SEED, 0, out=rt)      # out aliases residual
    assert_fp16(host(rt), ref, "aliased out=residual")
    # unaligned views (offset by one element) take the element-wise path
    big = torch.empty(rows * cols + 1, dtype=torch.float16, device="cuda")
    xv = big[1:].view(rows, cols)
    xv.copy_(dev(x))
    out = host(ls.bias_dropout_residual(xv, dev(b), dev(r), 0.1, SEED, 0))
    assert "scalar" in last_dispatch()
    assert_fp16(out, ref, "unaligned x")


@pytest.mark.parametrize("rows,cols", [(4096, 3072), (8192, 4096), (128, 1024), (37, 24), (5, 1000), (3, 13),
                                       (0, 8)])
@pytest.mark.parametrize("p", [0.1, 0.0, 1.0])
def test_bias_relu_dropout(ls, rows, cols, p):
    g = np.random.default_rng(rows * 7 + cols)
    x = synth.normal16(g, (rows, cols), 1.0)
    b = synth.normal16(g, (cols,), 0.02)
    out = host(ls.bias_relu_dropout(dev(x), dev(b), p, SEED, synth.SITE_FFN_ACT))
    ref = oracle.bias_relu_dropout(x, b, p, SEED, synth.SITE_FFN_ACT, BITS)
    assert_fp16(out, ref, f"bias_relu_dropout {rows}x{cols} p={p} [{last_dispatch()}]")


def test_nan_inf_propagate(ls):
    x = np.array([[np.nan, np.inf, -np.inf, 1.0, -1.0, 0.0, 2.0, 3.0]], np.float16)
    b = np.zeros(8, np.float16)
    out = host(ls.bias_relu_dropout(dev(x), dev(b), 0.0, 1, 0))
    ref = oracle.bias_relu_dropout(x, b, 0.0, 1, 0, BITS)
    assert_fp16(out, ref, "relu nan/inf")


# ----------------------------------------------------------------------------
# Backward of the fused elementwise operators
# ----------------------------------------------------------------------------

# full C3/C4 shapes, several 512-column segments with ragged last ones (384,
# 520, 768, 4104 columns), the element-wise path (cols % 8 != 0), one row,
# row counts that leave the last row group short
EW_BWD_SHAPES = [(4096, 768), (4096, 3072), (8192, 1024), (200, 384), (333, 768), (129, 520), (1000, 4104),
                 (37, 24), (1, 8), (3, 13), (300, 20), (17, 1)]


@pytest.mark.parametrize("rows,cols", EW_BWD_SHAPES)
@pytest.mark.parametrize("p", [0.1, 0.0, 1.0])
def test_bias_dropout_residual_bwd(ls, rows, cols, p):
    g = np.random.default_rng(rows * 7919 + cols)
    dy = synth.normal16(g, (rows, cols), 1.0)
    dx, db = ls.bias_dropout_residual_bwd(dev(dy), p, SEED, synth.SITE_FFN_OUT)
    what = f"bias_dropout_residual_bwd {rows}x{cols} p={p} [{last_dispatch()}]"
    ref_dx, ref_db = oracle.bias_dropout_residual_bwd(dy, p, SEED, synth.SITE_FFN_OUT, BITS)
    assert_fp16(host(dx), ref_dx, what + " dx")
    assert_fp16(host(db), ref_db, what + " dbias")


@pytest.mark.parametrize("rows,cols", EW_BWD_SHAPES)
def test_bias_relu_dropout_bwd_after_forward(ls, rows, cols):
    """GPU forward, then GPU backward from its output, against the oracle's
    backward written from the forward's inputs and mask."""
    g = np.random.default_rng(rows * 104729 + cols)
    x = synth.normal16(g, (rows, cols), 1.0)
    b = synth.normal16(g, (cols,), 0.02)
    dy = synth.normal16(g, (rows, cols), 1.0)
    p = 0.1
    out = ls.bias_relu_dropout(dev(x), dev(b), p, SEED, synth.SITE_FFN_ACT)
    dx, db = ls.bias_relu_dropout_bwd(dev(dy), out, p)
    what = f"bias_relu_dropout_bwd {rows}x{cols} [{last_dispatch()}]"
    ref_dx, ref_db = oracle.bias_relu_dropout_bwd(dy, x, b, p, SEED, synth.SITE_FFN_ACT, BITS)
    assert_fp16(host(dx), ref_dx, what + " dx")
    assert_fp16(host(db), ref_db, what + " dbias")


def test_ew_bwd_dispatch_alias_determinism_and_empty(ls):
    g = np.random.default_rng(5)
    dy = synth.normal16(g, (4096, 3072), 1.0)
    ref_dx, ref_db = oracle.bias_dropout_residual_bwd(dy, 0.1, SEED, 1, BITS)
    t = dev(dy)
    dx, db = ls.bias_dropout_residual_bwd(t, 0.1, SEED, 1, dx=t)          # in place
    assert last_dispatch().startswith("bias_dropout_residual_bwd/seg512_w16_g")
    assert_fp16(host(dx), ref_dx, "in-place dx")
    db2 = ls.bias_dropout_residual_bwd(dev(dy), 0.1, SEED, 1)[1]
    assert np.array_equal(host(db).view(np.uint16), host(db2).view(np.uint16))   # fixed order
    assert_fp16(host(db2), ref_db, "dbias")
    # the forward output may be overwritten by the gradient
    x = synth.normal16(g, (64, 768), 1.0)
    b = synth.normal16(g, (768,), 0.02)
    dy2 = synth.normal16(g, (64, 768), 1.0)
    out = ls.bias_relu_dropout(dev(x), dev(b), 0.1, SEED, 1)
    dx3, _ = ls.bias_relu_dropout_bwd(dev(dy2), out, 0.1, dx=out)
    assert_fp16(host(dx3), oracle.bias_relu_dropout_bwd(dy2, x, b, 0.1, SEED, 1, BITS)[0], "dx over out")
    # no rows: dbias is zero; no columns: nothing to do
    empty = torch.empty((0, 40), dtype=torch.float16, device="cuda")
    dbz = torch.full((40,), 3.0, dtype=torch.float16, device="cuda")
    ls.bias_dropout_residual_bwd(empty, 0.1, SEED, 1, dbias=dbz)
    assert (host(dbz) == 0).all()
    ls.bias_relu_dropout_bwd(empty, empty, 0.1, dbias=dbz)
    assert (host(dbz) == 0).all()


# ----------------------------------------------------------------------------
# Bias + Q/K/V head split and its backward (exact permutation: bit-exact)
# ----------------------------------------------------------------------------

# BERT-base (C3) and Transformer-big (C4) attention shapes, ragged segment
# counts, head_dim not a multiple of 8 (element-wise path), one token
QKV_SHAPES = [(32, 128, 12, 64), (32, 256, 16, 64), (3, 7, 5, 24), (2, 9, 3, 12), (1, 1, 1, 8), (4, 33, 2, 40)]


@pytest.mark.parametrize("batch,seq,heads,d", QKV_SHAPES)
def test_bias_qkv_split(ls, batch, seq, heads, d):
    g = np.random.default_rng(batch * 1009 + seq * 31 + heads * 7 + d)
    qkv = synth.normal16(g, (batch * seq, 3 * heads * d), 1.0)
    bias = synth.normal16(g, (3 * heads * d,), 0.02)
    out = host(ls.bias_qkv_split(dev(qkv), dev(bias), batch, seq, heads))
    what = f"bias_qkv_split {batch}x{seq}x{heads}x{d} [{last_dispatch()}]"
    ref = oracle.bias_qkv_split(qkv, bias, batch, seq, heads)
    assert np.array_equal(out.view(np.uint16), ref.view(np.uint16)), what
    dout = synth.normal16(g, ref.shape, 1.0)
    dq, db = ls.bias_qkv_split_bwd(dev(dout))
    what = f"bias_qkv_split_bwd {batch}x{seq}x{heads}x{d} [{last_dispatch()}]"
    ref_dq, ref_db = oracle.bias_qkv_split_bwd(dout, batch, seq, heads)
    assert np.array_equal(host(dq).view(np.uint16), ref_dq.view(np.uint16)), what
    assert_fp16(host(db), ref_db, what + " dbias")


def test_bias_qkv_split_dispatch_and_empty(ls):
    g = np.random.default_rng(3)
    qkv = dev(synth.normal16(g, (4096, 2304), 1.0))
    ls.bias_qkv_split(qkv, dev(synth.normal16(g, (2304,), 0.02)), 32, 128, 12)
    assert last_dispatch() == "bias_qkv_split/vec8"
    ls.bias_qkv_split_bwd(dev(synth.normal16(g, (3, 32, 12, 128, 64), 1.0)))
    assert last_dispatch().startswith("bias_qkv_split_bwd/seg512_w16_g")
    dbz = torch.full((3 * 2 * 8,), 5.0, dtype=torch.float16, device="cuda")
    ls.bias_qkv_split_bwd(torch.empty((3, 0, 2, 4, 8), dtype=torch.float16, device="cuda"), dbias=dbz)
    assert (host(dbz) == 0).all()


# ----------------------------------------------------------------------------
# Cross-entropy criterion
# ----------------------------------------------------------------------------

def assert_xent_rows(loss, lse, dx, x, y, eps, ignore, g, what):
    ref_loss, ref_lse = oracle.cross_entropy_fwd(x, y, eps, ignore)
    assert_fp32(lse, ref_lse, what + " lse", floor=1.0)
    assert_fp32(loss, ref_loss, what + " loss", floor=1.0)
    assert_fp16(dx, oracle.cross_entropy_bwd(x, y, eps, ignore, g), what + " dlogits")


def test_cross_entropy_c4_sampled_rows(ls):
    """Transformer-big criterion: logits [8192, 32768], Zipf targets, eps 0.1;
    every row computed on the GPU, the oracle on 1024 sampled rows, and on
    every row what holds at any size: max(x) <= lse <= max(x) + log V,
    loss >= 0 (lse bounds both the target logit and the mean logit), and
    the gradient row sums to zero (the softmax, the one-hot and the smoothing
    floor each sum to one) within its fp16 rounding."""
    T, V = synth.C4.tokens, synth.C4.vocab
    x = synth.criterion_logits(0, T)
    y = synth.criterion_targets()
    xd, yd = dev(x), dev(y)
    loss, lse = ls.cross_entropy_fwd(xd, yd, synth.CRITERION_SMOOTHING, -1)
    assert last_dispatch() == "cross_entropy_fwd/row_block512_v8"
    gs = synth.CRITERION_LOSS_SCALE / T           # mean over tokens, times the loss scale
    dx = ls.cross_entropy_bwd(xd, yd, lse, synth.CRITERION_SMOOTHING, -1, gs)
    assert last_dispatch() == "cross_entropy_bwd/vec8"
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(7).integers(0, T, 1021)]))
    hl, hs, hd = host(loss), host(lse), host(dx)
    assert_xent_rows(hl[rows], hs[rows], hd[rows], x[rows], y[rows],
                     synth.CRITERION_SMOOTHING, -1, gs, "cross_entropy C4")
    xmax = x.max(axis=1).astype(np.float64)
    lse64 = hs.astype(np.float64)
    assert np.all(lse64 >= xmax - 1e-6 * np.abs(xmax)), "lse below the row maximum"
    assert np.all(lse64 <= xmax + np.log(V) + 1e-5 * np.abs(xmax) + 1e-5), "lse above max + log V"
    assert np.all(hl.astype(np.float64) >= -1e-5 * np.maximum(np.abs(lse64), 1.0)), "negative loss"
    d64 = hd.astype(np.float64)
    rowsum = d64.sum(axis=1)
    # each element within half an fp16 spacing of its fp32 value, the fp32
    # values within a few ulps of exact: twice the spacings bounds the sum
    spacing = np.spacing(np.abs(hd)).astype(np.float64)
    bound = 2.0 * spacing.sum(axis=1) + 1e-6 * gs
    bad = np.abs(rowsum) > bound
    assert not bad.any(), f"gradient rows not summing to zero: {np.flatnonzero(bad)[:5]} {rowsum[bad][:5]}"


@pytest.mark.parametrize("rows,v", [(37, 1001), (5, 8), (1, 1), (3, 50257), (64, 4096), (17, 16392), (9, 2048)])
@pytest.mark.parametrize("eps", [0.0, 0.1])
def test_cross_entropy_shapes(ls, rows, v, eps):
    g = np.random.default_rng(rows * 131 + v)
    x = synth.normal16(g, (rows, v), 2.0)
    y = g.integers(0, v, size=rows).astype(np.int32)
    if rows > 2:
        y[1] = -100                              # ignored
    xd = dev(x)
    loss, lse = ls.cross_entropy_fwd(xd, dev(y), eps, -100)
    what = f"cross_entropy {rows}x{v} eps={eps} [{last_dispatch()}]"
    dx = ls.cross_entropy_bwd(xd, dev(y), lse, eps, -100, 0.5)
    assert_xent_rows(host(loss), host(lse), host(dx), x, y, eps, -100, 0.5, what)


def test_cross_entropy_nan_bad_target_alias(ls):
    g = np.random.default_rng(9)
    x = synth.normal16(g, (6, 1024), 1.0)
    x[2, 17] = np.nan
    x[3, 5] = np.inf
    y = np.array([3, 1024, 7, 8, -1, 0], np.int32)          # row 1: out of range; row 4: ignored
    xd = dev(x)
    loss, lse = ls.cross_entropy_fwd(xd, dev(y), 0.1, -1)
    lo = host(loss)
    assert np.isnan(lo[[1, 2, 3]]).all() and lo[4] == 0 and np.isfinite(lo[[0, 5]]).all()
    ref_loss, _ = oracle.cross_entropy_fwd(x, y, 0.1, -1)
    assert np.isnan(ref_loss[[1, 2, 3]]).all()
    dx = ls.cross_entropy_bwd(xd, dev(y), lse, 0.1, -1, 1.0, dlogits=xd)      # in place
    d = host(dx)
    assert np.isnan(d[1]).all() and (d[4] == 0).all()
    assert_fp16(d[[0, 5]], oracle.cross_entropy_bwd(x[[0, 5]], y[[0, 5]], 0.1, -1, 1.0), "in-place dlogits")


# ----------------------------------------------------------------------------
# HARS beam-search top-k (indices and scores bit-exact)
# ----------------------------------------------------------------------------

def check_topk(ls, lp, bs, k, what):
    s, i = ls.beam_topk(dev(lp), k, None if bs is None else dev(bs))
    ref_s, ref_i = oracle.hars_topk(lp, bs, k)
    got_i, got_s = host(i), host(s)
    assert np.array_equal(got_i, ref_i), f"{what}: ids {got_i[:2]} vs oracle {ref_i[:2]}"
    nan = np.isnan(ref_s)
    assert np.array_equal(np.isnan(got_s), nan), what                 # NaN payloads are not kept
    assert np.array_equal(got_s[~nan].view(np.uint32), ref_s[~nan].view(np.uint32)), what


def test_beam_topk_golden_example(ls):
    """The beam 2 x vocabulary 8 example of the HARS slides (fixture in
    tests/golden/): the kernel returns the oracle's top-k."""
    lp, k, _, _ = hars_example()
    check_topk(ls, lp, None, k, "beam_topk golden beam 2 x vocab 8")


def test_beam_topk_decoder_step(ls):
    """Transformer-big decoder step: 128 sentences x beam 4 over vocab 32768."""
    g = np.random.default_rng(17)
    logits = g.normal(size=(128, 4, 32768))
    lp = (logits - np.log(np.exp(logits).sum(-1, keepdims=True))).astype(np.float32)
    bs = np.cumsum(g.normal(-1.0, 0.5, size=(128, 4)), axis=1).astype(np.float32)
    check_topk(ls, lp, bs, 4, "beam_topk 128x4x32768")
    assert last_dispatch() == "beam_topk/hars_rows_block1024_merge"


@pytest.mark.parametrize("batch,beam,v,k", [(3, 2, 8, 2), (5, 1, 1, 1), (2, 3, 100003, 7), (4, 8, 50257, 8),
                                            (2, 4, 1000, 64), (3, 2, 600, 1000), (1, 16, 4096, 16),
                                            (2, 5, 33, 5), (7, 3, 32768, 3), (2, 4, 5000, 1024)])
def test_beam_topk_shapes(ls, batch, beam, v, k):
    g = np.random.default_rng(batch * 7 + beam * 13 + v + k)
    lp = g.normal(size=(batch, beam, v)).astype(np.float32)
    bs = g.normal(size=(batch, beam)).astype(np.float32) if beam > 1 else None
    check_topk(ls, lp, bs, k, f"beam_topk {batch}x{beam}x{v} k={k}")


def test_beam_topk_ties_special_values_and_overflow(ls):
    lp = np.zeros((2, 3, 40), np.float32)
    lp[0, 0, 1] = -0.0
    lp[0, 1, 4] = np.nan
    lp[0, 2, 5] = np.inf
    lp[1, :, ::7] = 3.0
    check_topk(ls, lp, None, 6, "ties and special values")
    # every candidate equal: all 131072 survive the threshold, more than the
    # survivor list holds, so the exact-pass fallback answers
    check_topk(ls, np.zeros((2, 4, 32768), np.float32), None, 4, "all equal")
    check_topk(ls, np.full((1, 2, 5000), -1.5, np.float32), np.zeros((1, 2), np.float32), 3, "all equal, small")


# ----------------------------------------------------------------------------
# LayerNorm
# ----------------------------------------------------------------------------

LN_SHAPES = [(128, 256), (4096, 768), (8192, 1024), (1000, 64), (77, 96), (33, 512), (9, 1536),
             (5, 2048), (3, 4096), (50, 100), (20, 13), (1, 8), (300, 768), (4, 4095),
             (300, 2047), (64, 3001), (1030, 767), (16384, 256), (4096, 1001)]


def ln_inputs(rows, h, seed):
    g = np.random.default_rng(seed)
    return (synth.normal16(g, (rows, h), 1.0), synth.uniform16(g, (h,), 0.5, 1.5),
            synth.normal16(g, (h,), 0.1), synth.normal16(g, (rows, h), 1.0))


@pytest.mark.parametrize("rows,h", LN_SHAPES)
def test_layernorm_fwd(ls, rows, h):
    x, gamma, beta, _ = ln_inputs(rows, h, rows + h)
    y, mean, rstd = ls.layernorm_fwd(dev(x), dev(gamma), dev(beta), synth.LN_EPS)
    ry, rmean, rrstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    tag = f"layernorm_fwd {rows}x{h} [{last_dispatch()}]"
    assert_fp16(host(y), ry, tag)
    sigma = 1.0 / rrstd.astype(np.float64)
    assert_fp32(host(mean), rmean, tag + " mean", floor=sigma)
    assert_fp32(host(rstd), rrstd, tag + " rstd")


@pytest.mark.parametrize("rows,h", LN_SHAPES)
def test_layernorm_bwd(ls, rows, h):
    x, gamma, beta, dy = ln_inputs(rows, h, rows * 3 + h)
    _, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    dx, dg, db = ls.layernorm_bwd(dev(dy), dev(x), dev(gamma), dev(mean), dev(rstd))
    rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, gamma, mean, rstd)
    tag = f"layernorm_bwd {rows}x{h} [{last_dispatch()}]"
    assert_fp16(host(dx), rdx, tag + " dx")
    assert_fp16(host(dg), rdg, tag + " dgamma")
    assert_fp16(host(db), rdb, tag + " dbeta")
    # the row kernel writes one partial row per block, and the finalisation
    # reads (clamped) up to as many rows as the workspace holds: the grid in
    # the dispatch name never exceeds that count
    grid = int(re.search(r"_g(\d+)$", last_dispatch()).group(1))
    assert 1 <= grid <= (ls.layernorm_bwd_workspace_bytes(rows, h) - 256) // (8 * h), tag
    # the column reduction has a fixed order: a second run is bit-identical
    dx2, dg2, db2 = ls.layernorm_bwd(dev(dy), dev(x), dev(gamma), dev(mean), dev(rstd))
    assert np.array_equal(host(dg2), host(dg)) and np.array_equal(host(db2), host(db))
    assert np.array_equal(host(dx2), host(dx))


LN_OFFSET_SHAPES = [(4096, 768), (448, 1024), (224, 256), (112, 96), (70, 4095), (56, 2048), (35, 13),
                    (140, 767)]


@pytest.mark.parametrize("rows,h", LN_OFFSET_SHAPES)
def test_layernorm_offset_rows(ls, rows, h):
    """Rows N(m, 1) with |m| / sigma in {0, 1, 3, 10, 30, 100, 1000}, both
    signs: the one-pass statistics meet the fp32 bar (the reduction runs over
    x minus the row's first element), and the outputs and the backward meet
    the fp16 bar."""
    g = np.random.default_rng(rows + 7 * h)
    x = synth.offset_rows16(g, rows, h)
    gamma = synth.uniform16(g, (h,), 0.5, 1.5)
    beta = synth.normal16(g, (h,), 0.1)
    dy = synth.normal16(g, (rows, h), 1.0)
    y, mean, rstd = ls.layernorm_fwd(dev(x), dev(gamma), dev(beta), synth.LN_EPS)
    ry, rmean, rrstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    tag = f"layernorm_fwd offset rows {rows}x{h} [{last_dispatch()}]"
    assert_fp16(host(y), ry, tag)
    sigma = 1.0 / rrstd.astype(np.float64)
    assert_fp32(host(mean), rmean, tag + " mean", floor=sigma)
    assert_fp32(host(rstd), rrstd, tag + " rstd")
    dx, dg, db = ls.layernorm_bwd(dev(dy), dev(x), dev(gamma), dev(rmean), dev(rrstd))
    rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, gamma, rmean, rrstd)
    tag = f"layernorm_bwd offset rows {rows}x{h} [{last_dispatch()}]"
    assert_fp16(host(dx), rdx, tag + " dx")
    assert_fp16(host(dg), rdg, tag + " dgamma")
    assert_fp16(host(db), rdb, tag + " dbeta")


def assert_fused_z(z, rz, tag):
    """The stored sum: the fp16 bar, and at most one element in 1000 rounded
    differently from the oracle at all (midpoint cases of the fp32 sum)."""
    assert_fp16(z, rz, tag + " z")
    differ = np.count_nonzero(np.asarray(z).view(np.uint16) != np.asarray(rz).view(np.uint16))
    assert differ <= max(1, np.asarray(z).size // 1000), f"{tag}: {differ} elements of z round differently"


FUSED_SHAPES = [(128, 256), (4096, 768), (8192, 1024), (77, 96), (33, 512), (9, 1536), (3, 4096), (20, 13),
                (1030, 767), (5, 2048), (300, 768), (1, 8), (16384, 256), (4, 4095), (45, 520), (33, 640),
                (1, 768)]


@pytest.mark.parametrize("rows,h", FUSED_SHAPES)
@pytest.mark.parametrize("p", [0.1, 0.0, 1.0])
def test_bias_dropout_residual_layernorm(ls, rows, h, p):
    """The fused sub-layer output block against the oracle, and bit for bit
    against the two separate operators called one after the other."""
    g = np.random.default_rng(rows * 7 + h)
    x, r = synth.normal16(g, (rows, h), 1.0), synth.normal16(g, (rows, h), 1.0)
    b = synth.normal16(g, (h,), 0.02)
    gamma, beta = synth.uniform16(g, (h,), 0.5, 1.5), synth.normal16(g, (h,), 0.1)
    eps, off = synth.LN_EPS, synth.SITE_ATTN_OUT
    z, y, mean, rstd = ls.bias_dropout_residual_layernorm(dev(x), dev(b), dev(r), dev(gamma), dev(beta), p, SEED,
                                                          off, eps)
    tag = f"bias_dropout_residual_layernorm {rows}x{h} p={p} [{last_dispatch()}]"
    rz, _, _, _ = oracle.bias_dropout_residual_layernorm(x, b, r, gamma, beta, p, SEED, off, BITS, eps)
    assert_fused_z(host(z), rz, tag)
    # An fp32 sum within 2^-24 of an fp16 rounding midpoint can round the
    # other way from the oracle's float64 sum (one element in ~4000): y and
    # the statistics are held to their bars against the oracle's LayerNorm of
    # the stored z, which is what the kernel normalises.
    ry, rmean, rrstd = oracle.layernorm_fwd(host(z), gamma, beta, eps)
    assert_fp16(host(y), ry, tag + " y")
    sigma = 1.0 / rrstd.astype(np.float64)
    assert_fp32(host(mean), rmean, tag + " mean", floor=sigma)
    assert_fp32(host(rstd), rrstd, tag + " rstd")
    # against the two standalone operators: z bit for bit; y and the
    # statistics to rounding (the fused kernel may give a row to fewer lanes,
    # so its fp32 sums run in another order)
    z2 = ls.bias_dropout_residual(dev(x), dev(b), dev(r), p, SEED, off)
    y2, mean2, rstd2 = ls.layernorm_fwd(z2, dev(gamma), dev(beta), eps)
    assert np.array_equal(host(z).view(np.uint16), host(z2).view(np.uint16)), tag + ": z differs from the separate op"
    assert_fp16(host(y), host(y2), tag + " y against the separate ops")
    assert_fp32(host(mean), host(mean2), tag + " mean against the separate ops", floor=sigma)
    assert_fp32(host(rstd), host(rstd2), tag + " rstd against the separate ops")


def test_bias_dropout_residual_layernorm_aliasing_offsets_and_empty(ls):
    """z written over the residual (in place) and over x; rows of the
    residual offset by up to 1000 sigma; no rows launches nothing; bad
    arguments are rejected before launching."""
    from non_gemm_amd import _lib
    rows, h, p, eps = 700, 768, 0.1, synth.LN_EPS
    g = np.random.default_rng(41)
    x = synth.normal16(g, (rows, h), 1.0)
    r = synth.offset_rows16(g, rows, h)
    b = synth.normal16(g, (h,), 0.02)
    gamma, beta = synth.uniform16(g, (h,), 0.5, 1.5), synth.normal16(g, (h,), 0.1)
    rz, _, _, _ = oracle.bias_dropout_residual_layernorm(x, b, r, gamma, beta, p, SEED, 2, BITS, eps)
    for target in ("residual", "x"):
        xt, rt = dev(x), dev(r)
        zt = rt if target == "residual" else xt
        z, y, mean, rstd = ls.bias_dropout_residual_layernorm(xt, dev(b), rt, dev(gamma), dev(beta), p, SEED, 2,
                                                              eps, z=zt)
        tag = f"fused, z aliasing {target} [{last_dispatch()}]"
        assert z.data_ptr() == zt.data_ptr()
        assert_fused_z(host(z), rz, tag)
        ry, rmean, rrstd = oracle.layernorm_fwd(host(z), gamma, beta, eps)     # LayerNorm of the stored z
        assert_fp16(host(y), ry, tag + " y")
        sigma = 1.0 / rrstd.astype(np.float64)
        assert_fp32(host(mean), rmean, tag + " mean", floor=sigma)
        assert_fp32(host(rstd), rrstd, tag + " rstd")
    e = torch.empty((0, h), dtype=torch.float16, device="cuda")
    ls.bias_dropout_residual_layernorm(e, dev(b), e, dev(gamma), dev(beta), p, SEED, 2, eps)
    assert last_dispatch() == "empty"
    lib = _lib.load()
    S = torch.cuda.current_stream().cuda_stream
    t = dev(x)
    for bad_p, bad_eps in ((1.5, eps), (0.1, 0.0)):
        rc = lib.ls_bias_dropout_residual_layernorm(t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                                    t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                                    t.data_ptr(), rows, h, bad_p, SEED, 2, bad_eps, S)
        assert rc == 3      # LS_ERR_PARAM


@pytest.mark.parametrize("rows,h,offset", [(4096, 768, 0), (300, 768, 1), (77, 96, 0), (5, 2048, 1), (1030, 767, 0),
                                           (8192, 1024, 0)])
def test_layernorm_bwd_split_calls(ls, rows, h, offset):
    """ls_layernorm_bwd_input then ls_layernorm_bwd_params, the second on
    another stream ordered by an event, give the combined call's results bit
    for bit (offset 1: dx one element into its buffer, so the element-wise
    path runs, whose block count differs from the vector path's)."""
    x, gamma, beta, dy = ln_inputs(rows, h, rows + 5 * h)
    _, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    args = (dev(dy), dev(x), dev(gamma), dev(mean), dev(rstd))
    dxbuf = torch.empty(rows * h + offset, dtype=torch.float16, device="cuda")
    dx_full = dxbuf[offset:].view(rows, h)
    ref = ls.layernorm_bwd(*args, dx=dx_full)
    ref = [host(t).copy() for t in ref]
    ws = torch.empty(ls.layernorm_bwd_workspace_bytes(rows, h), dtype=torch.uint8, device="cuda")
    dxbuf2 = torch.empty_like(dxbuf)
    dx = ls.layernorm_bwd_input(*args, ws, dx=dxbuf2[offset:].view(rows, h))
    tag = f"layernorm_bwd split {rows}x{h} [{last_dispatch()}]"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg, db = ls.layernorm_bwd_params(rows, h, ws)
    torch.cuda.current_stream().wait_stream(side)
    for a, b, what in ((dx, ref[0], "dx"), (dg, ref[1], "dgamma"), (db, ref[2], "dbeta")):
        assert np.array_equal(host(a).view(np.uint16), b.view(np.uint16)), f"{tag}: {what}"


def test_layernorm_bwd_params_batched(ls):
    """ls_layernorm_bwd_params_batched over 20 LayerNorms of mixed shapes
    (more than one launch's 16 jobs; a job with no rows, one with no
    columns): every job's dgamma / dbeta equal its own parameter call's bit
    for bit, and the oracle's to the fp16 bar."""
    shapes = [(4096, 768), (300, 768), (77, 96), (5, 2048), (1030, 767), (0, 768), (8192, 1024), (1, 8),
              (64, 0), (129, 520)]
    shapes = shapes + shapes[::-1]
    jobs, refs = [], []
    for i, (rows, h) in enumerate(shapes):
        if h == 0:
            jobs.append((rows, 0, None, None, None))
            refs.append(None)
            continue
        dg = torch.full((h,), 7.0, dtype=torch.float16, device="cuda")
        db = torch.full((h,), -7.0, dtype=torch.float16, device="cuda")
        if rows == 0:
            jobs.append((0, h, None, dg, db))
            refs.append((np.zeros(h, np.float16), np.zeros(h, np.float16), None, None))
            continue
        x, gamma, beta, dy = ln_inputs(rows, h, 300 + i)
        _, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
        args = (dev(dy), dev(x), dev(gamma), dev(mean), dev(rstd))
        ws = torch.empty(ls.layernorm_bwd_workspace_bytes(rows, h), dtype=torch.uint8, device="cuda")
        ls.layernorm_bwd_input(*args, ws)
        one = [host(t).copy() for t in ls.layernorm_bwd_params(rows, h, ws)]
        _, rdg, rdb = oracle.layernorm_bwd(dy, x, gamma, mean, rstd)
        jobs.append((rows, h, ws, dg, db))
        refs.append((one[0], one[1], rdg, rdb))
    out = ls.layernorm_bwd_params_batched(jobs)
    assert last_dispatch() == "layernorm_bwd_params/fixed_order_jobs18_launches2", last_dispatch()
    for (rows, h), (dg, db), ref in zip(shapes, out, refs):
        if ref is None:
            continue
        tag = f"batched params {rows}x{h}"
        assert np.array_equal(host(dg).view(np.uint16), ref[0].view(np.uint16)), tag + " dgamma"
        assert np.array_equal(host(db).view(np.uint16), ref[1].view(np.uint16)), tag + " dbeta"
        if ref[2] is not None:
            assert_fp16(host(dg), ref[2], tag + " dgamma vs oracle")
            assert_fp16(host(db), ref[3], tag + " dbeta vs oracle")


def test_layernorm_bwd_zero_rows_and_stale_header(ls):
    """No rows: dgamma and dbeta are the sums over no rows, zeros, from the
    combined call and from the parameter call alone (no workspace).  A
    workspace whose header no input call wrote: the count is clamped to what
    the workspace holds, so the call reads inside it (values unspecified)."""
    h = 768
    for call in ("combined", "params"):
        dg = torch.full((h,), 7.0, dtype=torch.float16, device="cuda")
        db = torch.full((h,), -7.0, dtype=torch.float16, device="cuda")
        if call == "combined":
            e = torch.empty((0, h), dtype=torch.float16, device="cuda")
            ls.layernorm_bwd(e, e, dev(np.ones(h, np.float16)), torch.empty(0, device="cuda"),
                             torch.empty(0, device="cuda"), dgamma=dg, dbeta=db)
        else:
            ls.layernorm_bwd_params(0, h, None, dgamma=dg, dbeta=db)
        assert np.all(host(dg) == 0) and np.all(host(db) == 0), call
    rows = 64
    ws = torch.full((ls.layernorm_bwd_workspace_bytes(rows, h),), 0x7F, dtype=torch.uint8, device="cuda")
    ls.layernorm_bwd_params(rows, h, ws)
    torch.cuda.synchronize()


def test_layernorm_bwd_workspace_reuse(ls):
    """One workspace serves calls of different shapes in turn (different
    block counts, so different partial-row layouts): each call is
    bit-identical to a call on a fresh workspace and matches the oracle."""
    shapes = [(4096, 768), (300, 768), (77, 96), (8192, 1024), (1, 8), (4096, 768)]
    need = max(ls.layernorm_bwd_workspace_bytes(r, h) for r, h in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")    # stale contents are ignored
    for i, (rows, h) in enumerate(shapes):
        x, gamma, beta, dy = ln_inputs(rows, h, 11 + i)
        _, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
        args = (dev(dy), dev(x), dev(gamma), dev(mean), dev(rstd))
        got = ls.layernorm_bwd(*args, workspace=ws)
        tag = f"layernorm_bwd reuse {rows}x{h} [{last_dispatch()}]"
        fresh = ls.layernorm_bwd(*args)
        for a, b in zip(got, fresh):
            assert np.array_equal(host(a), host(b)), tag
        rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, gamma, mean, rstd)
        assert_fp16(host(got[1]), rdg, tag + " dgamma")
        assert_fp16(host(got[2]), rdb, tag + " dbeta")


def test_layernorm_degenerate_rows(ls):
    """Constant rows give y = beta; rows (+a, -a, ...) the closed form."""
    h = 256
    x = np.zeros((4, h), np.float16)
    x[0] = 3.0
    x[1] = np.tile([0.5, -0.5], h // 2)
    x[2] = np.tile([100.0, -100.0], h // 2)
    gamma = np.ones(h, np.float16)
    beta = np.full(h, 0.25, np.float16)
    y, mean, rstd = ls.layernorm_fwd(dev(x), dev(gamma), dev(beta), synth.LN_EPS)
    ry, _, rrstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    assert_fp16(host(y), ry, "degenerate rows")
    assert np.all(host(y)[0] == np.float16(0.25)) and np.all(host(y)[3] == np.float16(0.25))


# ----------------------------------------------------------------------------
# Softmax
# ----------------------------------------------------------------------------

SM_SHAPES = [(8, 12, 128, 128), (32, 12, 128, 128), (32, 16, 256, 256), (2, 3, 17, 64),
             (2, 2, 9, 512), (1, 2, 5, 1024), (1, 1, 3, 2048), (1, 1, 3, 4096), (1, 2, 2, 8192),
             (1, 1, 2, 20000), (2, 2, 7, 100), (2, 3, 5, 7), (1, 1, 1, 1), (0, 12, 128, 128), (1, 2, 3, 1023),
             (3, 5, 9, 1000), (2, 3, 4, 2000)]


@pytest.mark.parametrize("shape", SM_SHAPES)
def test_softmax_fwd_dense(ls, shape):
    g = np.random.default_rng(sum(shape))
    x = synth.normal16(g, shape, 3.0)
    y = host(ls.softmax_fwd(dev(x)))
    ref = oracle.softmax_fwd(x)
    tag = f"softmax_fwd {shape} [{last_dispatch()}]"
    assert_fp16(y, ref, tag)
    if x.size:
        # argmax: compare where the oracle's row maximum is unique
        r = ref.reshape(-1, shape[-1]).astype(np.float64)
        yy = y.reshape(-1, shape[-1]).astype(np.float64)
        top = r.max(1, keepdims=True)
        unique = (r == top).sum(1) == 1
        assert np.array_equal(np.argmax(yy[unique], 1), np.argmax(r[unique], 1)), tag


@pytest.mark.parametrize("shape,name", [((8, 12, 128, 128), "lpr16_nch1_v8"), ((32, 12, 128, 128), "lpr8_nch2_v8"),
                                        ((2, 2, 33, 120), "lpr16_nch1_v8"), ((64, 8, 64, 72), "lpr8_nch2_v8")])
def test_softmax_row_mapping_follows_row_count(ls, shape, name):
    """Rows of 72-128 keys: 16 lanes x 1 vector while 8 x 2 would give fewer
    than 4096 waves (under 32768 rows), 8 x 2 from there on; same results
    either way, forward and backward."""
    g = np.random.default_rng(sum(shape) + 5)
    x = synth.normal16(g, shape, 3.0)
    y = host(ls.softmax_fwd(dev(x)))
    assert last_dispatch() == "softmax_fwd/" + name
    assert_fp16(y, oracle.softmax_fwd(x), f"softmax_fwd {shape} [{name}]")
    dy = synth.normal16(g, shape, 1.0)
    yv = oracle.softmax_fwd(x)
    k = shape[-1]
    dx = host(ls.softmax_bwd(dev(yv), dev(dy)))
    assert last_dispatch() == "softmax_bwd/" + name
    ref = oracle.softmax_bwd(yv.reshape(-1, k), dy.reshape(-1, k)).reshape(shape)
    assert_fp16(dx, ref, f"softmax_bwd {shape} [{name}]")


# the dense C2 case (no lengths, not causal) is the first of SM_SHAPES
@pytest.mark.parametrize("causal,with_lengths", [(False, True), (True, True), (True, False)])
def test_softmax_fwd_c2_masked(ls, causal, with_lengths):
    inp = synth.softmax_inputs()
    x, lens = inp["scores"], inp["key_lengths"]
    kl = lens if with_lengths else None
    y = host(ls.softmax_fwd(dev(x), dev(kl) if kl is not None else None, causal))
    ref = oracle.softmax_fwd(x, kl, causal)
    tag = f"softmax_fwd C2 causal={causal} lengths={with_lengths} [{last_dispatch()}]"
    assert_fp16(y, ref, tag)
    valid = oracle.ops.softmax_valid(*x.shape, kl, causal)
    assert np.all(y[~valid] == 0), tag + ": masked entries must be exactly 0"


@pytest.mark.parametrize("k", [64, 100, 128, 4096, 8192, 65536])
def test_softmax_fwd_edge_lengths(ls, k):
    """Key lengths 0, 1, ragged and beyond k (clamped); causal rows."""
    g = np.random.default_rng(k)
    b = 6
    x = synth.normal16(g, (b, 2, 5, k), 3.0)
    lens = np.array([0, 1, k // 2 + 3, k, k + 10, -4], np.int32)
    for causal in (False, True):
        y = host(ls.softmax_fwd(dev(x), dev(lens), causal))
        ref = oracle.softmax_fwd(x, lens, causal)
        assert_fp16(y, ref, f"softmax_fwd k={k} causal={causal} [{last_dispatch()}]")
        assert np.all(y[0] == 0) and np.all(y[5] == 0)


@pytest.mark.parametrize("shape", SM_SHAPES)
def test_softmax_bwd(ls, shape):
    g = np.random.default_rng(sum(shape) + 1)
    x = synth.normal16(g, shape, 3.0)
    yv = oracle.softmax_fwd(x)
    dy = synth.normal16(g, shape, 1.0)
    k = shape[-1]
    dx = host(ls.softmax_bwd(dev(yv), dev(dy)))
    ref = oracle.softmax_bwd(yv.reshape(-1, k), dy.reshape(-1, k)).reshape(shape)
    assert_fp16(dx, ref, f"softmax_bwd {shape} [{last_dispatch()}]")


def test_softmax_bwd_c2_masked_and_alias(ls):
    inp = synth.softmax_inputs()
    yv = oracle.softmax_fwd(inp["scores"], inp["key_lengths"], True)
    dy = inp["grad_out"]
    k = yv.shape[-1]
    dyt = dev(dy)
    ls.softmax_bwd(dev(yv), dyt, dx=dyt)          # dx aliases dy
    ref = oracle.softmax_bwd(yv.reshape(-1, k), dy.reshape(-1, k)).reshape(yv.shape)
    out = host(dyt)
    assert_fp16(out, ref, "softmax_bwd C2 aliased")
    assert np.all(out[yv == 0] == 0)


# ----------------------------------------------------------------------------
# Embedding
# ----------------------------------------------------------------------------

def test_embedding_c4(ls):
    inp = synth.embedding_inputs()
    ids, E, P, s = inp["ids"], inp["tok_emb"], inp["pos_emb"], inp["scale"]
    p, off = synth.DROPOUT_P, synth.SITE_EMBEDDING
    out = host(ls.embedding_fwd(dev(ids), dev(E), dev(P), s, p, SEED, off))
    ref = oracle.embedding_fwd(ids, E, P, s, p, SEED, off, BITS)
    assert_fp16(out, ref, f"embedding_fwd C4 [{last_dispatch()}]")
    v, h = E.shape
    dE = torch.full((v, h), 7.0, dtype=torch.float32, device="cuda")     # zero_first must clear it
    ls.embedding_bwd(dev(ids), dev(inp["grad_out"]), dE, s, p, SEED, off, zero_first=True)
    got = host(dE)
    want = oracle.embedding_bwd(ids, inp["grad_out"], v, s, p, SEED, off, BITS)
    # fp32 atomics sum in no fixed order: bound by 1e-5 of the sum of |terms|
    keep = oracle.dropout_keep(ids.size * h, p, SEED, off, BITS).reshape(-1, h)
    terms = np.abs(s * inp["grad_out"].astype(np.float64) * keep * oracle.dropout_scale(p, BITS))
    mag = np.zeros((v, h))
    np.add.at(mag, ids.reshape(-1), terms)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(err <= 1e-5 * mag + 1e-30), f"embedding_bwd [{last_dispatch()}]: max err {err.max()}"
    untouched = np.setdiff1d(np.arange(v), ids)
    assert np.all(got[untouched] == 0)
    assert "sorted1024" in last_dispatch()


def _emb_bwd_check(ls, ids, dy, v, s, p, seed, off, acc=None, what=""):
    h = dy.shape[-1]
    dE = dev(acc.copy()) if acc is not None else torch.zeros((v, h), dtype=torch.float32, device="cuda")
    ls.embedding_bwd(dev(ids), dev(dy), dE, s, p, seed, off, zero_first=acc is None)
    got = host(dE).astype(np.float64)
    want = oracle.embedding_bwd(ids, dy, v, s, p, seed, off, BITS, grad_in=acc).astype(np.float64)
    keep = oracle.dropout_keep(ids.size * h, p, seed, off, BITS).reshape(-1, h)
    terms = np.abs(s * dy.astype(np.float64).reshape(-1, h) * keep * oracle.dropout_scale(p, BITS))
    mag = np.zeros((v, h)) if acc is None else np.abs(acc.astype(np.float64))
    ok_ids = (ids.reshape(-1) >= 0) & (ids.reshape(-1) < v)
    np.add.at(mag, ids.reshape(-1)[ok_ids], terms[ok_ids])
    err = np.abs(got - want)
    assert np.all(err <= 1e-5 * mag + 1e-30), f"{what} [{last_dispatch()}]: max err {err.max()}"
    return last_dispatch()


@pytest.mark.parametrize("counts,h", [([1], 768), ([64], 768), ([65], 1024), ([2000], 768),
                                      ([31, 33, 97, 1], 520), ([7] * 40, 1536), ([16, 17, 15], 512),
                                      ([1500, 700, 3], 64), ([1] * 1100, 8)])
def test_embedding_bwd_repeated_ids(ls, counts, h):
    """Runs of one id inside and across the 16 sorted positions of a wave, the
    64 of a block and the 1024 tokens of a sorted chunk; column slices with a
    ragged last slice (520, 1536 columns)."""
    g = np.random.default_rng(sum(counts) + h)
    ids = np.concatenate([np.full(c, 5 + 3 * i, np.int32) for i, c in enumerate(counts)])
    ids = g.permutation(ids)
    pad = (-ids.size) % 4
    ids = np.concatenate([ids, np.full(pad, 2, np.int32)]).reshape(4, -1)
    dy = synth.normal16(g, (ids.size, h), 1.0)
    disp = _emb_bwd_check(ls, ids, dy, max(300, 5 + 3 * len(counts)), 32.0, 0.1, 21, 3, what=f"counts {counts} h={h}")
    assert "sorted1024" in disp


def test_embedding_bwd_other_paths(ls):
    g = np.random.default_rng(4)
    ids = g.integers(0, 50, size=(40, 500)).astype(np.int32)          # 20000 tokens
    dy = synth.normal16(g, (ids.size, 64), 1.0)
    _emb_bwd_check(ls, ids, dy, 50, 2.0, 0.1, 9, 3, what="20000 tokens")
    ids = g.integers(0, 9, size=(3, 11)).astype(np.int32)             # hidden not a multiple of 8
    dy = synth.normal16(g, (ids.size, 20), 1.0)
    assert "elementwise" in _emb_bwd_check(ls, ids, dy, 9, 2.0, 0.0, 9, 3, what="hidden 20")
    # The widest vocabulary of the sorted path (ids in 22 bits, below the
    # no-key marker) and the first one past it (64-token chunks sorted by one
    # wave with 64-bit keys); the largest id repeats across chunks.
    for v, path in (((1 << 22) - 1, "sorted1024"), (1 << 22, "chunk64")):
        ids = g.integers(0, v, size=(3, 700)).astype(np.int32)
        ids[0, :50] = v - 1
        ids[2, 100:400:3] = v - 1
        ids[1, 5] = -1
        dy = synth.normal16(g, (ids.size, 8), 1.0)
        assert path in _emb_bwd_check(ls, ids, dy, v, 2.0, 0.1, 9, 3, what=f"vocab {v}")


@pytest.mark.parametrize("b,l,h,v", [(2, 7, 64, 50), (3, 5, 768, 100), (1, 33, 24, 9), (2, 4, 20, 11),
                                     (4, 16, 1024, 3), (1, 1, 8, 1), (1, 40, 2048, 64)])
def test_embedding_small(ls, b, l, h, v):
    g = np.random.default_rng(b * l * h)
    ids = g.integers(0, v, size=(b, l)).astype(np.int32)
    E = synth.normal16(g, (v, h), 0.2)
    P = synth.normal16(g, (l + 2, h), 0.5)
    dy = synth.normal16(g, (b * l, h), 1.0)
    for p in (0.1, 0.0):
        out = host(ls.embedding_fwd(dev(ids), dev(E), dev(P), 4.0, p, 9, 3))
        assert_fp16(out, oracle.embedding_fwd(ids, E, P, 4.0, p, 9, 3, BITS), f"embedding_fwd {b,l,h,v} p={p}")
        acc = synth.normal16(g, (v, h), 1.0).astype(np.float32)
        dE = dev(acc.copy())
        ls.embedding_bwd(dev(ids), dev(dy), dE, 4.0, p, 9, 3, zero_first=False)     # accumulate
        want = oracle.embedding_bwd(ids, dy, v, 4.0, p, 9, 3, BITS, grad_in=acc)
        np.testing.assert_allclose(host(dE), want, rtol=1e-5, atol=1e-4,
                                   err_msg=f"embedding_bwd {b,l,h,v} p={p} [{last_dispatch()}]")


def test_embedding_invalid_ids(ls):
    v, h = 10, 64
    ids = np.array([[0, 10, -1, 9, 3, 1000]], np.int32)
    E = np.ones((v, h), np.float16)
    P = np.zeros((6, h), np.float16)
    out = host(ls.embedding_fwd(dev(ids), dev(E), dev(P), 1.0, 0.0, 1, 0))
    assert np.all(np.isnan(out[[1, 2, 5]])) and np.all(out[[0, 3, 4]] == 1)
    dy = np.ones((6, h), np.float16)
    dE = torch.zeros((v, h), dtype=torch.float32, device="cuda")
    ls.embedding_bwd(dev(ids), dev(dy), dE, 1.0, 0.0, 1, 0, zero_first=True)
    got = host(dE)
    assert np.all(got[[0, 3, 9]] == 1) and np.all(got[[1, 2, 4, 5, 6, 7, 8]] == 0)


# ----------------------------------------------------------------------------
# Adam over the workspace
# ----------------------------------------------------------------------------

def fp16_ulp(x):
    """Spacing of fp16 numbers at x (subnormal spacing below 2^-14)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_adam_update(p_gpu, p_ref, p0, tag, ulps=2, rare_ulps=10, rare_frac=1e-5):
    """The update itself, p - p0, against the oracle's: within `ulps` fp16
    spacings of the parameter (each step rounds p to fp16; fp32 and float64
    arithmetic may round a step differently now and then).  A parameter whose
    step lies next to a rounding midpoint, where the fp32 result rounded to
    fp16 (two roundings) and the float64 one fall on different sides, can do
    so at every step (the workload's gradient is the same at every step), so
    at most `rare_frac` of the parameters may differ by up to `rare_ulps`
    spacings (each result stays within half a spacing per step of the exact
    path: ten steps, ten spacings apart at most).  A step that is missing,
    halved, doubled or of the wrong sign moves every p by many spacings
    (lr = 1e-4 is ~6 spacings at |p| = 0.02 per step) and fails."""
    d_gpu = np.asarray(p_gpu, np.float64) - np.asarray(p0, np.float64)
    d_ref = np.asarray(p_ref, np.float64) - np.asarray(p0, np.float64)
    sp = fp16_ulp(np.maximum(np.abs(np.asarray(p_ref, np.float64)), np.abs(np.asarray(p0, np.float64))))
    diff = np.abs(d_gpu - d_ref)
    bad = ~(diff <= ulps * sp)
    worst = ~(diff <= rare_ulps * sp)
    if worst.any() or bad.sum() > rare_frac * bad.size:
        i = int(np.argwhere(worst if worst.any() else bad)[0][0])
        raise AssertionError(f"{tag}: update of {int(bad.sum())}/{bad.size} parameters off by more than {ulps} "
                             f"fp16 spacings ({int(worst.sum())} by more than {rare_ulps}); first at {i}: "
                             f"{d_gpu[i]} vs oracle {d_ref[i]} (p0 {p0[i]})")
    moved = np.count_nonzero(d_ref)
    assert moved == 0 or np.count_nonzero(d_gpu) >= 0.9 * moved, f"{tag}: parameters left unchanged"


@pytest.mark.parametrize("n,decoupled,offset,steps", [(1_000_003, True, 0, 10), (77, True, 0, 10),
                                                      (50_001, True, 3, 10), (4096, False, 0, 1),
                                                      (4096, False, 0, 10), (2052, True, 0, 3)])
def test_adam_steps(ls, n, decoupled, offset, steps):
    """AdamW (the workspace trainer's mode): moments depend on the gradient
    only, so they meet the fp32 bar over all ten steps.  L2 mode feeds the
    fp16 parameter back into the gradient; once a parameter's fp16 rounding
    differs by one ulp between fp32 and fp64 arithmetic, its moments differ by
    up to wd * ulp, so after the first step only the parameter is compared."""
    g = np.random.default_rng(n)
    p = synth.normal16(g, (n,), 0.02)
    gr = synth.normal16(g, (n,), 1e-3)
    hp = dict(synth.ADAM_HYPER)
    hp["decoupled_wd"] = decoupled
    # offset > 0: views that are not 16-byte aligned take the element-wise path
    pt = torch.empty(n + offset, dtype=torch.float16, device="cuda")[offset:]
    pt.copy_(dev(p))
    gt = dev(gr)
    mt = torch.zeros(n + offset, dtype=torch.float32, device="cuda")[offset:]
    vt = torch.zeros(n + offset, dtype=torch.float32, device="cuda")[offset:]
    rp, rm, rv = p, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for step in range(1, steps + 1):
        ls.adam_workspace_step(pt, gt, mt, vt, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"], step, hp["grad_scale"], decoupled)
        rp, rm, rv = oracle.adam_workspace_step(rp, gr, rm, rv, hp["lr"], hp["beta1"], hp["beta2"],
                                                hp["eps"], hp["weight_decay"], step, hp["grad_scale"],
                                                decoupled)
    tag = f"adam n={n} steps={steps} [{last_dispatch()}]"
    assert_fp16(host(pt), rp, tag + " param")
    assert_adam_update(host(pt), rp, p, tag)
    if decoupled or steps == 1:
        assert_fp32(host(mt), rm, tag + " exp_avg")
        assert_fp32(host(vt), rv, tag + " exp_avg_sq")


@pytest.mark.parametrize("decoupled", [True, False])
def test_adam_large_steps(ls, decoupled):
    """lr 1e-2 and weight decay 0.1: every step moves a parameter by far more
    than the fp16 bar, so the parameter values themselves pin the update
    (sign, size, bias corrections, the weight-decay form) over ten steps."""
    n = 20_011
    g = np.random.default_rng(77 + decoupled)
    p = synth.normal16(g, (n,), 0.5)
    gr = synth.normal16(g, (n,), 1e-2)
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.98, eps=1e-8, weight_decay=0.1, grad_scale=1.0)
    pt, gt = dev(p), dev(gr)
    mt, vt = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    rp, rm, rv = p, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for step in range(1, 11):
        ls.adam_workspace_step(pt, gt, mt, vt, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"],
                               step, hp["grad_scale"], decoupled)
        rp, rm, rv = oracle.adam_workspace_step(rp, gr, rm, rv, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                                hp["weight_decay"], step, hp["grad_scale"], decoupled)
    tag = f"adam lr 1e-2 decoupled={decoupled} [{last_dispatch()}]"
    assert_fp16(host(pt), rp, tag + " param")
    assert_adam_update(host(pt), rp, p, tag)
    assert np.mean(np.abs(rp.astype(np.float64) - p.astype(np.float64)) > 0.05) > 0.9     # the steps are large


def test_adam_full_workspace_sampled(ls):
    """The 350M-parameter workspace of the Adam workload, ten single-launch
    steps on the GPU; the oracle (element-wise) on 4M sampled parameters,
    chunk boundaries and the last element included.  Every parameter is also
    held to what the workload's constant gradient fixes in closed form: with
    zero-initialised moments and the same g' = g / grad_scale at every step,
    m_t = (1 - beta1^t) g' and v_t = (1 - beta2^t) g'^2 (so the
    bias-corrected step is lr * (g' / (|g'| + eps) + wd * p) each time), and
    after ten steps p is within five fp16 spacings (half a spacing per step,
    along a monotone path) of p0 - 10 lr (g' / (|g'| + eps) + wd p0)."""
    n = synth.C5_PARAMS
    nchunks = -(-n // synth.C5_CHUNK)
    p = np.empty(n, np.float16)
    gr = np.empty(n, np.float16)
    for c in range(nchunks):
        pc, gc = synth.adam_chunk(c)
        lo, hi = c * synth.C5_CHUNK, min(n, (c + 1) * synth.C5_CHUNK)
        p[lo:hi], gr[lo:hi] = pc[:hi - lo], gc[:hi - lo]
    hp = synth.ADAM_HYPER
    pt, gt = dev(p), dev(gr)
    mt, vt = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    idx = np.unique(np.concatenate([np.random.default_rng(5).integers(0, n, 4_000_000),
                                    np.arange(0, n, synth.C5_CHUNK), [n - 1, n - 8, 7, 8]]))
    rp, rg = p[idx], gr[idx]
    rm, rv = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    for step in range(1, synth.ADAM_STEPS + 1):
        ls.adam_workspace_step(pt, gt, mt, vt, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"], step, hp["grad_scale"], hp["decoupled_wd"])
        rp, rm, rv = oracle.adam_workspace_step(rp, rg, rm, rv, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                                hp["weight_decay"], step, hp["grad_scale"], hp["decoupled_wd"])
    ti = torch.from_numpy(idx).cuda()
    tag = f"adam 350M sampled [{last_dispatch()}]"
    assert_fp16(host(pt[ti]), rp, tag + " param")
    assert_adam_update(host(pt[ti]), rp, p[idx], tag)
    assert_fp32(host(mt[ti]), rm, tag + " exp_avg")
    assert_fp32(host(vt[ti]), rv, tag + " exp_avg_sq")
    assert hp["decoupled_wd"], "the closed form below assumes a gradient that does not depend on p"
    t = synth.ADAM_STEPS
    c1, c2 = 1.0 - hp["beta1"] ** t, 1.0 - hp["beta2"] ** t
    for lo in range(0, n, synth.C5_CHUNK):
        hi = min(n, lo + synth.C5_CHUNK)
        g1 = gr[lo:hi].astype(np.float64) / hp["grad_scale"]
        p0 = p[lo:hi].astype(np.float64)
        m_cf, v_cf = c1 * g1, c2 * g1 * g1
        assert_fp32(host(mt[lo:hi]), m_cf, f"adam 350M closed-form exp_avg [{lo}, {hi})")
        assert_fp32(host(vt[lo:hi]), v_cf, f"adam 350M closed-form exp_avg_sq [{lo}, {hi})")
        p10 = host(pt[lo:hi])
        pred = p0 - t * hp["lr"] * (g1 / (np.abs(g1) + hp["eps"]) + hp["weight_decay"] * p0)
        top = np.maximum(np.abs(p0), np.abs(p10.astype(np.float64))).astype(np.float16)
        tol = 5.0 * np.spacing(top).astype(np.float64) + 1e-7
        err = np.abs(p10.astype(np.float64) - pred)
        bad = err > tol
        assert not bad.any(), (f"adam 350M closed-form params [{lo}, {hi}): {bad.sum()} off, "
                               f"first at {lo + np.flatnonzero(bad)[0]}: {err[bad][0]} > {tol[bad][0]}")


def test_adam_resume_bit_identical(ls):
    """5 steps, save, reload, 5 more == 10 straight steps, bit for bit."""
    from non_gemm_amd import workspace
    g = np.random.default_rng(3)
    shapes = [(768, 768), (768,), (3072, 768), (13,)]
    base = [synth.normal16(g, s, 0.02) for s in shapes]
    grads = [synth.normal16(g, s, 1e-3) for s in shapes]

    def make():
        ps = [torch.nn.Parameter(dev(b.copy())) for b in base]
        ws = workspace.link(ps)
        for pp, gg in zip(ps, grads):
            pp.grad.copy_(dev(gg))
        return ps, ws
    hp = dict(lr=1e-4, betas=(0.9, 0.98), eps=1e-8, weight_decay=0.01)
    ps1, ws1 = make()
    for _ in range(10):
        ws1.step(**hp)
    ps2, ws2 = make()
    for _ in range(5):
        ws2.step(**hp)
    state = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in ws2.state_dict().items()}
    ps3, ws3 = make()
    ws3.load_state_dict({k: (v.cuda() if torch.is_tensor(v) else v) for k, v in state.items()})
    for _ in range(5):
        ws3.step(**hp)
    assert torch.equal(ws1.param, ws3.param)
    assert torch.equal(ws1.exp_avg, ws3.exp_avg) and torch.equal(ws1.exp_avg_sq, ws3.exp_avg_sq)
    # parameters are views of the workspace
    assert torch.equal(ps3[2].detach().reshape(-1), ws3.param[ws3.offsets[2]:ws3.offsets[2] + 3072 * 768])


# ----------------------------------------------------------------------------
# Bandwidth reference kernels (measurement only): exact copy, per-KiB sums
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 4096, 4096 * 5 + 48, 1 << 24])
def test_probe_copy_and_read(ls, nbytes):
    from non_gemm_amd import _lib
    lib = _lib.load()
    S = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(nbytes)
    src_np = rng.standard_normal(nbytes // 4).astype(np.float32)
    src = dev(src_np)
    dst = torch.full_like(src, float("nan"))
    _lib.check("ls_probe_copy", lib.ls_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, S))
    assert np.array_equal(host(dst).view(np.uint32), src_np.view(np.uint32))
    nsink = -(-nbytes // 1024)
    sink = torch.full((nsink + 4,), -7.0, dtype=torch.float32, device="cuda")
    _lib.check("ls_probe_read", lib.ls_probe_read(sink.data_ptr(), src.data_ptr(), nbytes, S))
    got = host(sink)
    pad = np.zeros(nsink * 256, np.float64)
    pad[:src_np.size] = src_np
    want = pad.reshape(nsink, 256).sum(axis=1)
    scale = np.abs(pad).reshape(nsink, 256).sum(axis=1)
    assert np.all(np.abs(got[:nsink] - want) <= 1e-5 * scale + 1e-30)
    assert np.all(got[nsink:] == -7.0)        # nothing written past ceil(bytes / 1024)


# ----------------------------------------------------------------------------
# HIP graph replay: the chain's launches captured once and replayed, with
# eager work and synchronisation between replays; every replay must equal the
# eager result bit for bit (no memset nodes, no state carried between calls)
# ----------------------------------------------------------------------------

CHAIN_CONFIGS = [(1, synth.C1), (3, synth.C3), (4, synth.C4)]


@pytest.mark.parametrize("config,shape", CHAIN_CONFIGS, ids=["tiny-128x256", "bert-base", "transformer-big"])
def test_layer_chain_configs(ls, config, shape):
    """A configured layer chain end to end, from the config's seeded inputs:
    every GPU operator consumes the GPU outputs of the one before it, the
    oracle its own outputs (dropout 0.1 at the three sites, LayerNorm eps
    1e-5), and every output is held to the fp16 / fp32 bars."""
    inp = synth.chain_inputs(shape, config=config)
    p, eps = synth.DROPOUT_P, synth.LN_EPS
    g = {k: dev(v) for k, v in inp.items()}
    probs = ls.softmax_fwd(g["scores"])
    a = ls.bias_dropout_residual(g["attn_proj"], g["attn_bias"], g["residual"], p, SEED, synth.SITE_ATTN_OUT)
    l1, m1, r1 = ls.layernorm_fwd(a, g["gamma1"], g["beta1"], eps)
    act = ls.bias_relu_dropout(g["ffn_pre"], g["ffn_bias1"], p, SEED, synth.SITE_FFN_ACT)
    f = ls.bias_dropout_residual(g["ffn_proj"], g["ffn_bias2"], l1, p, SEED, synth.SITE_FFN_OUT)
    l2, m2, r2 = ls.layernorm_fwd(f, g["gamma2"], g["beta2"], eps)
    dx2, dg2, db2 = ls.layernorm_bwd(g["grad_y2"], f, g["gamma2"], m2, r2)
    dx1, dg1, db1 = ls.layernorm_bwd(g["grad_y1"], a, g["gamma1"], m1, r1)
    dprobs = ls.softmax_bwd(probs, g["grad_probs"])

    k = shape.seq
    o_probs = oracle.softmax_fwd(inp["scores"])
    o_a = oracle.bias_dropout_residual(inp["attn_proj"], inp["attn_bias"], inp["residual"], p, SEED,
                                       synth.SITE_ATTN_OUT, BITS)
    o_l1, o_m1, o_r1 = oracle.layernorm_fwd(o_a, inp["gamma1"], inp["beta1"], eps)
    o_act = oracle.bias_relu_dropout(inp["ffn_pre"], inp["ffn_bias1"], p, SEED, synth.SITE_FFN_ACT, BITS)
    o_f = oracle.bias_dropout_residual(inp["ffn_proj"], inp["ffn_bias2"], o_l1, p, SEED, synth.SITE_FFN_OUT, BITS)
    o_l2, o_m2, o_r2 = oracle.layernorm_fwd(o_f, inp["gamma2"], inp["beta2"], eps)
    o_dx2, o_dg2, o_db2 = oracle.layernorm_bwd(inp["grad_y2"], o_f, inp["gamma2"], o_m2, o_r2)
    o_dx1, o_dg1, o_db1 = oracle.layernorm_bwd(inp["grad_y1"], o_a, inp["gamma1"], o_m1, o_r1)
    o_dprobs = oracle.softmax_bwd(o_probs.reshape(-1, k), inp["grad_probs"].reshape(-1, k)).reshape(o_probs.shape)

    tag = f"chain config {config} ({shape.name})"
    for name, got, ref in (("softmax fwd", probs, o_probs), ("attention bias+dropout+residual", a, o_a),
                           ("LayerNorm 1", l1, o_l1), ("bias+ReLU+dropout", act, o_act),
                           ("FFN bias+dropout+residual", f, o_f), ("LayerNorm 2", l2, o_l2),
                           ("LayerNorm 2 dx", dx2, o_dx2), ("LayerNorm 2 dgamma", dg2, o_dg2),
                           ("LayerNorm 2 dbeta", db2, o_db2), ("LayerNorm 1 dx", dx1, o_dx1),
                           ("LayerNorm 1 dgamma", dg1, o_dg1), ("LayerNorm 1 dbeta", db1, o_db1),
                           ("softmax bwd", dprobs, o_dprobs)):
        assert_fp16(host(got), ref, f"{tag}: {name}")
    chain_stats_bar(f"{tag}: LayerNorm 1", host(a), o_a, host(m1), host(r1), o_m1, o_r1)
    chain_stats_bar(f"{tag}: LayerNorm 2", host(f), o_f, host(m2), host(r2), o_m2, o_r2)


def chain_stats_bar(tag, x, o_x, mean, rstd, o_mean, o_rstd):
    """LayerNorm statistics inside a chain.  Rows whose input is bit-identical
    on both sides are held to the 1e-5 bar.  A row whose input differs (an
    fp16 rounding upstream that went the other way, within the fp16 bar)
    moves the statistics by the first-order change that difference causes:
    d mean = sum(dx) / H, d rstd = -rstd^3 * sum((x - mean) * dx) / H; such
    rows get the bar plus twice that change.  An fp32 result falls within
    2^-24 of an fp16 rounding midpoint about once in 2^12 elements, so the
    differing inputs must stay below 1e-3 of all elements."""
    xg, xr = x.astype(np.float64), o_x.astype(np.float64)
    differ = xg != xr
    assert differ.mean() < 1e-3, f"{tag}: {int(differ.sum())} of {differ.size} inputs differ"
    same = ~differ.any(axis=1)
    om, ors = o_mean.astype(np.float64), o_rstd.astype(np.float64)
    sigma = 1.0 / ors
    assert_fp32(mean[same], o_mean[same], tag + " mean", floor=sigma[same])
    assert_fp32(rstd[same], o_rstd[same], tag + " rstd")
    if (~same).any():
        d = (xg - xr)[~same]
        h = x.shape[1]
        d_mean = np.abs(d.sum(axis=1)) / h
        d_rstd = ors[~same] ** 3 * np.abs(((xr[~same] - om[~same, None]) * d).sum(axis=1)) / h
        gm, gr = mean[~same].astype(np.float64), rstd[~same].astype(np.float64)
        assert (np.abs(gm - om[~same]) <= 1e-5 * np.maximum(np.abs(om[~same]), sigma[~same]) + 2 * d_mean).all(), \
            tag + " mean (rows with differing input)"
        assert (np.abs(gr - ors[~same]) <= 1e-5 * ors[~same] + 2 * d_rstd).all(), tag + " rstd (rows with differing input)"


def test_graph_replay_matches_eager(ls):
    g = np.random.default_rng(77)
    T, H, F = 256, 768, 3072
    x = dev(synth.normal16(g, (T, H), 1.0))
    r = dev(synth.normal16(g, (T, H), 1.0))
    b = dev(synth.normal16(g, (H,), 0.02))
    gm = dev(synth.uniform16(g, (H,), 0.5, 1.5))
    bt = dev(synth.normal16(g, (H,), 0.1))
    f = dev(synth.normal16(g, (T, F), 1.0))
    fb = dev(synth.normal16(g, (F,), 0.02))
    dy = dev(synth.normal16(g, (T, H), 1.0))
    sc = dev(synth.normal16(g, (2, 12, 128, 128), 1.0))
    out = {k: torch.empty_like(v) for k, v in (("z", x), ("y", x), ("a", f), ("dx", x), ("s", sc), ("ds", sc))}
    mean, rstd = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    dg, db = torch.empty(H, dtype=torch.float16, device="cuda"), torch.empty(H, dtype=torch.float16, device="cuda")
    ws = torch.empty(ls.layernorm_bwd_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    ids = dev(g.integers(0, 500, size=(2, 128)).astype(np.int32))
    dE = torch.empty((500, H), dtype=torch.float32, device="cuda")
    edy = dev(synth.normal16(g, (256, H), 1.0))
    # the fused block and the LayerNorm backward as its input call plus the
    # batched parameter call (two LayerNorms' workspaces)
    out.update({k: torch.empty_like(x) for k in ("z2", "y2", "dx2", "dx3")})
    mean2, rstd2 = torch.empty(T, device="cuda"), torch.empty(T, device="cuda")
    pg = {k: torch.empty(H, dtype=torch.float16, device="cuda") for k in ("dg2", "db2", "dg3", "db3")}
    ws2, ws3 = torch.empty_like(ws), torch.empty_like(ws)

    def step():
        ls.bias_dropout_residual(x, b, r, 0.1, SEED, 0, out=out["z"])
        ls.layernorm_fwd(out["z"], gm, bt, 1e-5, y=out["y"], mean=mean, rstd=rstd)
        ls.bias_relu_dropout(f, fb, 0.1, SEED, 1, out=out["a"])
        ls.layernorm_bwd(dy, out["z"], gm, mean, rstd, dx=out["dx"], dgamma=dg, dbeta=db, workspace=ws)
        ls.softmax_fwd(sc, y=out["s"])
        ls.softmax_bwd(out["s"], sc, dx=out["ds"])
        ls.embedding_bwd(ids, edy, dE, 16.0, 0.1, SEED, 3, zero_first=True)
        ls.bias_dropout_residual_layernorm(x, b, r, gm, bt, 0.1, SEED, 2, 1e-5, z=out["z2"], y=out["y2"],
                                           mean=mean2, rstd=rstd2)
        ls.layernorm_bwd_input(dy, out["z2"], gm, mean2, rstd2, ws2, dx=out["dx2"])
        ls.layernorm_bwd_input(out["y2"], out["z"], gm, mean, rstd, ws3, dx=out["dx3"])
        ls.layernorm_bwd_params_batched([(T, H, ws2, pg["dg2"], pg["db2"]), (T, H, ws3, pg["dg3"], pg["db3"])])

    def snap():
        torch.cuda.synchronize()
        return [t.clone() for t in (*out.values(), mean, rstd, dg, db, mean2, rstd2, *pg.values(), dE)]

    step()
    ref = snap()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for rep in range(3):
        for t in (*out.values(), mean, rstd, dg, db, mean2, rstd2, *pg.values(), dE):
            t.fill_(7)                         # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        got = snap()
        for i, (a, e) in enumerate(zip(got[:-1], ref[:-1])):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.float16 else a.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.float16 else e.view(torch.int32)), \
                f"replay {rep}: output {i} differs from the eager run"
        # the embedding gradient adds with atomics in no fixed order: equal up to fp32 rounding
        assert torch.allclose(got[-1], ref[-1], rtol=1e-5, atol=1e-4), f"replay {rep}: embedding gradient"


def test_graph_replay_other_entry_points(ls):
    """The remaining entry points captured in one HIP graph: every replay
    (with eager work between replays) is bit-identical to the eager run.
    Adam updates its buffers in place, so they are reset before each run."""
    g = np.random.default_rng(78)
    T, H, F, V = 256, 768, 3072, 4096
    B, L, NH = 2, 128, 12
    ids = dev(g.integers(0, 500, size=(B, L)).astype(np.int32))
    E = dev(synth.normal16(g, (500, H), 0.02))
    P = dev(synth.sinusoid_table(L, H))
    dy = dev(synth.normal16(g, (T, H), 1.0))
    dyf = dev(synth.normal16(g, (T, F), 1.0))
    act = torch.relu(dev(synth.normal16(g, (T, F), 1.0)))
    qkv = dev(synth.normal16(g, (T, 3 * H), 1.0))
    qb = dev(synth.normal16(g, (3 * H,), 0.02))
    dqo = dev(synth.normal16(g, (3, B, NH, L, H // NH), 1.0))
    logits = dev(synth.normal16(g, (64, V), 2.0))
    tgt = dev(g.integers(0, V, size=64).astype(np.int32))
    lp = dev(g.normal(size=(4, 4, 2000)).astype(np.float32))
    bs = dev(g.normal(size=(4, 4)).astype(np.float32))
    p0 = dev(synth.normal16(g, (100_003,), 0.02))
    gr = dev(synth.normal16(g, (100_003,), 1e-3))
    m0 = torch.zeros(100_003, device="cuda")
    f16 = dict(dtype=torch.float16, device="cuda")
    o = {"emb": torch.empty((T, H), **f16), "dx1": torch.empty((T, H), **f16), "db1": torch.empty(H, **f16),
         "dx2": torch.empty((T, F), **f16), "db2": torch.empty(F, **f16),
         "qs": torch.empty((3, B, NH, L, H // NH), **f16), "dq": torch.empty((T, 3 * H), **f16),
         "dqb": torch.empty(3 * H, **f16), "loss": torch.empty(64, device="cuda"),
         "lse": torch.empty(64, device="cuda"), "dl": torch.empty((64, V), **f16),
         "ts": torch.empty((4, 4), device="cuda"), "ti": torch.empty((4, 4), dtype=torch.int32, device="cuda"),
         "p": torch.empty_like(p0), "m": torch.empty_like(m0), "v": torch.empty_like(m0)}
    u8 = dict(dtype=torch.uint8, device="cuda")
    ws1 = torch.empty(max(ls.elementwise_bwd_workspace_bytes(T, H), 16), **u8)
    ws2 = torch.empty(max(ls.elementwise_bwd_workspace_bytes(T, F), 16), **u8)
    ws3 = torch.empty(max(ls.elementwise_bwd_workspace_bytes(T, 3 * H), 16), **u8)
    from non_gemm_amd import _lib
    ws4 = torch.empty(max(_lib.load().ls_beam_topk_workspace_bytes(4, 4, 4), 16), **u8)
    hp = synth.ADAM_HYPER

    def reset_adam():
        o["p"].copy_(p0)
        o["m"].copy_(m0)
        o["v"].copy_(m0)

    def step():
        ls.embedding_fwd(ids, E, P, 27.7, 0.1, SEED, 3, out=o["emb"])
        ls.bias_dropout_residual_bwd(dy, 0.1, SEED, 2, dx=o["dx1"], dbias=o["db1"], workspace=ws1)
        ls.bias_relu_dropout_bwd(dyf, act, 0.1, dx=o["dx2"], dbias=o["db2"], workspace=ws2)
        ls.bias_qkv_split(qkv, qb, B, L, NH, out=o["qs"])
        ls.bias_qkv_split_bwd(dqo, dqkv=o["dq"], dbias=o["dqb"], workspace=ws3)
        ls.cross_entropy_fwd(logits, tgt, 0.1, -1, loss=o["loss"], lse=o["lse"])
        ls.cross_entropy_bwd(logits, tgt, o["lse"], 0.1, -1, 1.0 / 64, dlogits=o["dl"])
        ls.beam_topk(lp, 4, bs, top_scores=o["ts"], top_ids=o["ti"], workspace=ws4)
        ls.adam_workspace_step(o["p"], gr, o["m"], o["v"], hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"], 3, 1.0, True)

    def snap():
        torch.cuda.synchronize()
        return {k: t.clone() for k, t in o.items()}

    reset_adam()
    step()
    ref = snap()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    reset_adam()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for rep in range(3):
        for k, t in o.items():
            t.fill_(3)                         # eager work between replays
        reset_adam()
        torch.cuda.synchronize()
        graph.replay()
        got = snap()
        for k in o:
            assert torch.equal(got[k].view(torch.int16) if got[k].dtype == torch.float16 else got[k],
                               ref[k].view(torch.int16) if ref[k].dtype == torch.float16 else ref[k]) or \
                (got[k].dtype == torch.float32 and torch.equal(got[k].view(torch.int32), ref[k].view(torch.int32))), \
                f"replay {rep}: {k} differs from the eager run"


def test_timed_launch_same_result_and_events(ls):
    """ls_time_next_launch: the armed launch gives the same output, its events
    measure a positive duration, and the next call runs untimed."""
    from non_gemm_amd import _lib
    lib = _lib.load()
    g = np.random.default_rng(12)
    x = dev(synth.normal16(g, (4096, 3072), 1.0))
    b = dev(synth.normal16(g, (3072,), 0.02))
    ref = host(ls.bias_relu_dropout(x, b, 0.1, SEED, 1))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()                  # torch creates its events on first use
    torch.cuda.synchronize()
    assert lib.ls_time_next_launch(e0.cuda_event, e1.cuda_event) == 0
    out = ls.bias_relu_dropout(x, b, 0.1, SEED, 1)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint16), ref.view(np.uint16))
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 10.0
    out2 = ls.bias_relu_dropout(x, b, 0.1, SEED, 1)        # disarmed: plain launch
    assert np.array_equal(host(out2).view(np.uint16), ref.view(np.uint16))

    # the LayerNorm backward's row kernel takes the same hook
    xs, gamma, beta, dy = ln_inputs(4096, 768, 5)
    _, mean, rstd = oracle.layernorm_fwd(xs, gamma, beta, synth.LN_EPS)
    args = (dev(dy), dev(xs), dev(gamma), dev(mean), dev(rstd))
    ref_ln = [host(t) for t in ls.layernorm_bwd(*args)]
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    f1.record()
    torch.cuda.synchronize()
    assert lib.ls_time_next_launch(f0.cuda_event, f1.cuda_event) == 0
    got = [host(t) for t in ls.layernorm_bwd(*args)]
    torch.cuda.synchronize()
    for a_, b_ in zip(got, ref_ln):
        assert np.array_equal(a_.view(np.uint16), b_.view(np.uint16))
    assert 0.0 < f0.elapsed_time(f1) < 10.0
    # a call rejected before launching disarms the events: the next call runs
    # untimed
    assert lib.ls_time_next_launch(f0.cuda_event, f1.cuda_event) == 0 and lib.ls_time_armed() == 1
    with pytest.raises(_lib.LsError):
        ls.layernorm_fwd(dev(xs), dev(gamma), dev(beta), 0.0)       # eps <= 0: rejected, nothing launched
    assert lib.ls_time_armed() == 0
    got = [host(t) for t in ls.layernorm_bwd(*args)]
    for a_, b_ in zip(got, ref_ln):
        assert np.array_equal(a_.view(np.uint16), b_.view(np.uint16))


@pytest.mark.parametrize("k", [16384, 65536])
def test_softmax_longest_rows_fwd_bwd(ls, k):
    """The block-per-row path up to its largest row (65536 keys)."""
    g = np.random.default_rng(k + 1)
    x = synth.normal16(g, (1, 1, 3, k), 3.0)
    y = ls.softmax_fwd(dev(x))
    assert_fp16(host(y), oracle.softmax_fwd(x, None, False), f"softmax_fwd k={k} [{last_dispatch()}]")
    dy = synth.normal16(g, (3, k), 1.0)
    yr = oracle.softmax_fwd(x, None, False).reshape(3, k)
    dx = ls.softmax_bwd(dev(yr), dev(dy))
    assert_fp16(host(dx), oracle.softmax_bwd(yr, dy), f"softmax_bwd k={k} [{last_dispatch()}]")
