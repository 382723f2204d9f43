"""Host model of the column-sum backward kernels' addressing (CPU only).

The kernels' index arithmetic, restated with NumPy over every block, wave,
lane and row step that a launch runs, for every shape the GPU tests and the
benchmark use: each load and store of ew_bwd_vec_kernel (dy, out, dx),
colsum_block_fold (the partial rows and its LDS slots) and
colsum_finalize_kernel (the partial rows, d_bias) falls inside its buffer,
and the workspace the library asks for holds every partial row.  The launch
geometry (row groups) comes from the library itself, through
ls_elementwise_bwd_workspace_bytes.

The same model shows what a variant that loads all of a wave's rows before
the first wait needs: without a bound on the row index (r < r_end) its loads
run past the last row of dy at the benchmark's own shape.
"""
import numpy as np
import pytest

from non_gemm_amd import _lib

WAVE, WAVES = 64, 16                    # lanes per wave, waves per 1024-thread block
SEG_VECS = 64                           # 16-byte vectors per column segment (512 columns)
FIN_COLS, FIN_SLICES, FIN_LOADS = 32, 32, 8   # finalisation block: 32 columns x 32 slices, 8 loads per thread

SHAPES = [(4096, 768), (4096, 3072), (8192, 1024), (8192, 4096), (200, 384), (333, 768), (129, 520),
          (1000, 4104), (7, 8), (1, 8), (37, 24), (4096, 2304), (8192, 3072), (5, 1000), (3, 13), (64, 64)]


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def geometry(lib, rows, cols):
    ws = lib.ls_elementwise_bwd_workspace_bytes(rows, cols)
    assert ws > 0 and ws % (4 * cols) == 0
    groups = ws // (4 * cols)
    return groups, -(-rows // groups), ws


def vec_kernel_accesses(rows, cols, groups, rpg):
    """Vector indices (16-byte units) that ew_bwd_vec_kernel loads from dy / out
    and stores to dx, and the partial-row elements colsum_block_fold writes."""
    nv = cols // 8
    gx = -(-nv // SEG_VECS)
    bx, by, wave, lane = np.meshgrid(np.arange(gx), np.arange(groups), np.arange(WAVES), np.arange(WAVE),
                                     indexing="ij")
    cv = bx * SEG_VECS + lane                             # this lane's vector column
    col_ok = cv < nv
    r_begin = by * rpg
    r_end = np.minimum(rows, r_begin + rpg)
    touched = []
    r = r_begin + wave
    # first row's loads, then per step: the next row's loads (guarded by rn < r_end), this row's store
    first = col_ok & (r < r_end)
    touched.append(r[first] * nv + cv[first])
    while True:
        live = r < r_end
        if not live.any():
            break
        rn = r + WAVES
        nxt = col_ok & live & (rn < r_end)
        touched.append(rn[nxt] * nv + cv[nxt])
        st = col_ok & live
        touched.append(r[st] * nv + cv[st])
        r = np.where(live, rn, r)
    vec = np.concatenate(touched) if touched else np.zeros(0, np.int64)
    # colsum_block_fold: thread c < 512 of block (bx, by) writes column bx*512 + c of row by, if < cols
    c = np.arange(SEG_VECS * 8)
    bxx, byy, cc = np.meshgrid(np.arange(gx), np.arange(groups), c, indexing="ij")
    col = bxx * SEG_VECS * 8 + cc
    ok = col < cols
    part = byy[ok] * cols + col[ok]
    # its LDS slots fold[wave][half][lane] (float4): lane = c >> 3 < 64, half = (c & 7) >> 2 < 2
    assert (c >> 3).max() < WAVE and ((c & 7) >> 2).max() < 2
    return vec, part


def finalize_accesses(cols, groups):
    """Partial-row elements colsum_finalize_kernel reads and d_bias elements it writes."""
    gx = -(-cols // FIN_COLS)
    bx, sl, cl, i = np.meshgrid(np.arange(gx), np.arange(FIN_SLICES), np.arange(FIN_COLS), np.arange(FIN_LOADS),
                                indexing="ij")
    c = bx * FIN_COLS + cl
    g = sl + i * FIN_SLICES
    # every thread loads at clamped indices (the values past the rows or
    # columns are masked after they arrive); with no groups nothing is read
    reads = (np.minimum(g, groups - 1) * cols + np.minimum(c, cols - 1)).ravel() if groups else np.zeros(0, int)
    # slice 0 of each block writes its 32 columns
    writes = (np.arange(gx)[:, None] * FIN_COLS + np.arange(FIN_COLS)[None, :]).ravel()
    writes = writes[writes < cols]
    return reads, writes


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_column_sum_backward_stays_in_bounds(lib, rows, cols):
    groups, rpg, ws = geometry(lib, rows, cols)
    assert groups <= FIN_SLICES * FIN_LOADS     # the finalisation's loads per thread cover every row
    part_elems = ws // 4
    reads, writes = finalize_accesses(cols, groups)
    assert reads.size and reads.min() >= 0 and reads.max() < part_elems
    assert writes.min() >= 0 and writes.max() < cols
    assert np.unique(writes).size == cols       # every d_bias element written exactly by one thread
    if cols % 8 == 0:
        nv_total = rows * cols // 8
        vec, part = vec_kernel_accesses(rows, cols, groups, rpg)
        assert vec.min() >= 0 and vec.max() < nv_total, (vec.min(), vec.max(), nv_total)
        assert part.min() >= 0 and part.max() < part_elems
        # every row of every column segment is visited (nothing is skipped)
        assert np.unique(vec).size == nv_total
        # every partial element of every group is written
        assert np.unique(part).size == groups * cols
    else:
        # element-wise kernel: thread = column c < cols of group by; rows [by*rpg, min(rows, by*rpg+rpg))
        c = np.arange(-(-cols // 256) * 256)
        c = c[c < cols]
        last = np.minimum(rows, (groups - 1) * rpg + rpg) - 1
        assert last * cols + c.max() < rows * cols
        assert (groups - 1) * cols + c.max() < part_elems


def test_unbounded_batched_row_loads_would_run_past_dy(lib):
    """A variant loading all of a wave's rows (up to 4) before its first wait,
    with the row index bounded by the group's row count but not by r_end, at
    the benchmark's bias+dropout+residual backward [4096, 768]: the last row
    group's waves reach rows past the tensor's end."""
    rows, cols = 4096, 768
    groups, rpg, _ = geometry(lib, rows, cols)
    nv = cols // 8
    per_wave = -(-rpg // WAVES)                  # rows a wave owns
    batch = 4                                     # rows loaded at once in the variant
    assert per_wave <= batch
    # rows a wave would load: r_begin + wave + 16 k, k < batch, with no r < r_end test
    r_begin = np.arange(groups)[:, None, None] * rpg
    r = r_begin + np.arange(WAVES)[None, :, None] + WAVES * np.arange(batch)[None, None, :]
    assert r.max() >= rows                        # past the last row
    overrun_bytes = (r.max() - rows + 1) * nv * 16
    assert overrun_bytes > 0
