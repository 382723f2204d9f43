"""Host model of the LayerNorm backward's partial-row addressing (CPU only).

The row kernel stores each block's column sums (2h floats: the dgamma then
the dbeta columns) in tiles of 32 columns: column c of block b at
t0 * slots + b * wt + (c - t0), where t0 = c rounded down to a multiple of
32, wt = min(32, 2h - t0), and slots = the partial rows the workspace holds.
The finalisation kernel reads column c of block b at the same index, with b
and c clamped into range.  Restated here with NumPy for every shape the GPU
tests and the benchmark use (slots from the library itself, through
ls_layernorm_bwd_workspace_bytes): the stores fill the workspace's partial
area exactly once each, every read lands on the store of the same
(block, column), and a finalisation block's 32 columns are one contiguous run.
"""
import numpy as np
import pytest

from non_gemm_amd import _lib

HEADER = 256          # bytes ahead of the partial rows
TILE = 32             # columns per tile
FIN_SLICES, FIN_LOADS = 32, 8

SHAPES = [(4096, 768), (8192, 1024), (1000, 768), (37, 1000), (5000, 4096), (300, 3), (129, 2050),
          (512, 1023), (65, 100), (3000, 130), (1, 8), (7, 17), (256, 4096), (255, 2), (128, 256)]


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def store_index(b, c, slots, w):
    t0 = c // TILE * TILE
    wt = np.minimum(TILE, w - t0)
    return t0 * slots + b * wt + (c - t0)


@pytest.mark.parametrize("rows,h", SHAPES)
def test_partial_tiles_cover_the_workspace_once(lib, rows, h):
    ws = lib.ls_layernorm_bwd_workspace_bytes(rows, h)
    w = 2 * h
    assert (ws - HEADER) % (4 * w) == 0
    slots = (ws - HEADER) // (4 * w)
    assert 1 <= slots <= 256
    b, c = np.meshgrid(np.arange(slots), np.arange(w), indexing="ij")
    idx = store_index(b, c, slots, w)
    # every (block, column) has its own float, and together they are the whole area
    assert idx.min() == 0 and idx.max() == slots * w - 1
    assert np.unique(idx).size == slots * w

    # the finalisation: block k takes tile k, thread (slice s, column cl) loads
    # blocks s + 32 i (i < 8) at clamped indices, then keeps those below the count
    for k in range(-(-w // TILE)):
        t0 = k * TILE
        cl, s, i = np.meshgrid(np.arange(TILE), np.arange(FIN_SLICES), np.arange(FIN_LOADS), indexing="ij")
        cc = np.minimum(t0 + cl, w - 1)
        bb = np.minimum(s + FIN_SLICES * i, slots - 1)
        rd = t0 * slots + bb * min(TILE, w - t0) + (cc - t0)
        assert rd.min() >= 0 and rd.max() < slots * w
        kept = (t0 + cl < w) & (s + FIN_SLICES * i < slots)
        np.testing.assert_array_equal(rd[kept], store_index(bb[kept], cc[kept], slots, w))
        # one contiguous run per block: the tile's slots rows of wt columns
        wt = min(TILE, w - t0)
        assert np.array_equal(np.unique(rd[kept]), np.arange(t0 * slots, t0 * slots + slots * wt))
