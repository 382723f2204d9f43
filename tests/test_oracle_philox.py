"""Pins for the oracle's Philox4x32-10 and its dropout decisions (CPU only)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox
from oracle.ops import dropout_keep, dropout_scale, drop_threshold

HERE = os.path.dirname(os.path.abspath(__file__))
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    """Compile the rocRAND-header reference program for the host."""
    hdr = os.path.join(ROCM_INC, "rocrand", "rocrand_philox4x32_10.h")
    if shutil.which("g++") is None or not os.path.exists(hdr):
        pytest.skip("g++ or rocRAND headers unavailable")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC,
                    os.path.join(HERE, "philox_ref.cpp"), "-o", exe], check=True)

    def run(requests):
        text = "".join(f"{s} {sub} {skip} {n}\n" for s, sub, skip, n in requests)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [np.array([int(w, 16) for w in line.split()], dtype=np.uint64)
                for line in out.strip().split("\n")]
    return run


@pytest.mark.parametrize("seed,stream,first_block", [
    (0, 0, 0),
    (0x0123456789ABCDEF, 0, 0),
    (0x0123456789ABCDEF, 3, 0),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 12345),
    (42, 7, (5 << 32) + 2),          # counter word 1 non-zero
    (0xDEADBEEF, 1 << 40, (1 << 33) - 3),   # stream word 3 non-zero; word-0 carry
])
def test_philox_matches_rocrand_engine(rocrand_ref, seed, stream, first_block):
    """rocRAND's engine with (seed, subsequence=stream, discard=4*block) walks
    the counter (block, block>>32, lo(stream), hi(stream)) with key
    (lo(seed), hi(seed)) and returns the four words of each call in order."""
    nblocks = 64
    ref = rocrand_ref([(seed, stream, 4 * first_block, 4 * nblocks)])[0]
    blocks = np.arange(first_block, first_block + nblocks, dtype=np.uint64)
    ours = philox.philox_words(blocks, seed, stream).reshape(-1)
    np.testing.assert_array_equal(ours, ref)


def test_field_order_low_first():
    """16- and 8-bit fields are the 32-bit words cut from the low end up."""
    n = 4096
    w32 = philox.random_fields(np.arange(n // 2), 32, 9, 2)
    w16 = philox.random_fields(np.arange(n), 16, 9, 2)
    w8 = philox.random_fields(np.arange(2 * n), 8, 9, 2)
    np.testing.assert_array_equal(w16[0::2] | (w16[1::2] << np.uint64(16)), w32)
    w8_16 = w8[0::2] | (w8[1::2] << np.uint64(8))
    np.testing.assert_array_equal(w8_16, w16)


def test_sparse_and_dense_index_agree():
    idx = np.array([7, 1_000_003, 5, 6, 1 << 36], dtype=np.uint64)
    dense = philox.random_fields(np.arange(64), 16, 11, 4)
    sparse = philox.random_fields(idx, 16, 11, 4)
    assert sparse[0] == dense[7] and sparse[2] == dense[5] and sparse[3] == dense[6]
    one = philox.random_fields(np.array([1 << 36], dtype=np.uint64), 16, 11, 4)
    assert one[0] == sparse[4]


@pytest.mark.parametrize("bits", [8, 16, 32])
def test_keep_rate_binomial(bits):
    """Keep fraction within 5 sigma of Binomial(n, 1 - p_eff)."""
    n = 3_145_728                      # one [4096, 768] tensor
    p = 0.1
    keep = dropout_keep(n, p, 0x0123456789ABCDEF, 0, bits)
    q = 1.0 - drop_threshold(p, bits) / float(1 << bits)
    sigma = np.sqrt(n * q * (1 - q))
    assert abs(keep.sum() - n * q) < 5 * sigma


def test_threshold_and_scale_edge_cases():
    assert drop_threshold(0.0, 16) == 0
    assert drop_threshold(1.0, 16) == 65536
    assert drop_threshold(0.1, 16) == 6553           # floor(0.1f * 65536)
    assert drop_threshold(0.1, 8) == 25
    assert dropout_scale(1.0, 16) == 0.0
    assert dropout_scale(0.0, 16) == 1.0
    assert dropout_scale(0.5, 16) == 2.0
    assert dropout_keep(1000, 0.0, 1, 0, 16).all()
    assert not dropout_keep(1000, 1.0, 1, 0, 16).any()
    with pytest.raises(ValueError):
        dropout_keep(10, 1.5, 1, 0, 16)


def test_sites_and_neighbours_uncorrelated():
    """Chi-square on 2-bit pairs (keep_a, keep_b) at p = 0.5: different stream
    words, different seeds and neighbouring elements look independent."""
    n = 1 << 18
    a = dropout_keep(n, 0.5, 77, 0, 16)
    others = [dropout_keep(n, 0.5, 77, 1, 16), dropout_keep(n, 0.5, 78, 0, 16), np.roll(a, 1)]
    for b in others:
        counts = np.bincount(a.astype(int) * 2 + b.astype(int), minlength=4)
        expected = n / 4.0
        chi2 = ((counts - expected) ** 2 / expected).sum()
        assert chi2 < 25.0, chi2           # 3 dof; p ~ 1.5e-5
