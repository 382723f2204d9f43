"""The allocation-free LayerNorm backward (ls_layernorm_bwd_noalloc) through
the C ABI, against the workspace entry point (ls_layernorm_bwd) on the same
inputs: two calls in a row, the second smaller, so the second reuses the
static scratch the first left behind; plus the oracle's bar, the size limit
and the empty case."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import fp16_mismatch

pytestmark = pytest.mark.gpu

LS_OK, LS_ERR_WORKSPACE = 0, 4


def _inputs(rows, h, seed):
    g = np.random.default_rng(seed)
    x = synth.normal16(g, (rows, h), 1.0)
    gamma = synth.uniform16(g, (h,), 0.5, 1.5)
    beta = synth.normal16(g, (h,), 0.1)
    dy = synth.normal16(g, (rows, h), 1.0)
    _, mean, rstd = oracle.layernorm_fwd(x, gamma, beta, synth.LN_EPS)
    return dy, x, gamma, mean, rstd


def test_noalloc_layernorm_bwd_matches_workspace_entry_point():
    from non_gemm_amd import _lib
    lib = _lib.load()
    S = torch.cuda.current_stream().cuda_stream
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    assert lib.ls_layernorm_bwd_noalloc_max_bytes() == 256 + (2 << 20)
    for i, (rows, h) in enumerate([(4096, 768), (300, 96)]):         # the second call is smaller
        dy, x, gamma, mean, rstd = _inputs(rows, h, 31 + i)
        t = [d(a) for a in (dy, x, gamma, mean, rstd)]
        outs = []
        for which in ("noalloc", "workspace"):
            dx = torch.empty((rows, h), dtype=torch.float16, device="cuda")
            dg = torch.full((h,), 7.0, dtype=torch.float16, device="cuda")
            db = torch.full((h,), 7.0, dtype=torch.float16, device="cuda")
            ptrs = [dx.data_ptr(), dg.data_ptr(), db.data_ptr()] + [a.data_ptr() for a in t]
            if which == "noalloc":
                rc = lib.ls_layernorm_bwd_noalloc(*ptrs, rows, h, S)
            else:
                nbytes = lib.ls_layernorm_bwd_workspace_bytes(rows, h)
                ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                rc = lib.ls_layernorm_bwd(*ptrs, rows, h, ws.data_ptr(), nbytes, S)
            assert rc == LS_OK, (which, rc, lib.ls_last_error())
            torch.cuda.synchronize()
            outs.append([o.cpu().numpy() for o in (dx, dg, db)])
        tag = f"layernorm_bwd_noalloc {rows}x{h} call {i + 1}"
        for a, b, what in zip(outs[0], outs[1], ("dx", "dgamma", "dbeta")):
            assert not fp16_mismatch(a, b).any(), f"{tag}: {what} differs from ls_layernorm_bwd"
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"{tag}: {what} not bit-identical"
        rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, gamma, mean, rstd)
        for a, b, what in zip(outs[0], (rdx, rdg, rdb), ("dx", "dgamma", "dbeta")):
            assert not fp16_mismatch(a, b).any(), f"{tag}: {what} vs the oracle"


def test_noalloc_layernorm_bwd_limits():
    from non_gemm_amd import _lib
    lib = _lib.load()
    S = torch.cuda.current_stream().cuda_stream
    fake = ctypes.c_void_p(0x1000)                  # never reached: the size check comes first
    rc = lib.ls_layernorm_bwd_noalloc(*([fake] * 8), 4096, 2048, S)
    assert rc == LS_ERR_WORKSPACE and b"scratch" in lib.ls_last_error()
    # no rows: dgamma and dbeta are zeros, nothing else is touched
    h = 512
    dg = torch.full((h,), 3.0, dtype=torch.float16, device="cuda")
    db = torch.full((h,), 3.0, dtype=torch.float16, device="cuda")
    rc = lib.ls_layernorm_bwd_noalloc(None, dg.data_ptr(), db.data_ptr(), None, None, None, None, None, 0, h, S)
    assert rc == LS_OK
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(db == 0)
