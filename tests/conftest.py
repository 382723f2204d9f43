import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def fp16_mismatch(a, b, atol=2e-3, rtol=1e-2):
    """Boolean mask of fp16 elements that fail the parity bar.

    An element fails iff |a - b| > atol AND |a - b| > rtol * |b|, with b the
    oracle value (both bounds at once would be unsatisfiable near zero).
    NaN must match NaN; infinities must match exactly.
    """
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    same_inf = np.isinf(a) & np.isinf(b) & (a == b)
    with np.errstate(invalid="ignore"):
        d = np.abs(a - b)
        bad = (d > atol) & (d > rtol * np.abs(b))
    bad |= np.isnan(a) ^ np.isnan(b)
    return bad & ~both_nan & ~same_inf


@pytest.fixture
def assert_fp16_close():
    import numpy as np

    def check(a, b, what="", atol=2e-3, rtol=1e-2):
        bad = fp16_mismatch(a, b, atol, rtol)
        if bad.any():
            idx = np.argwhere(bad)[:5]
            af = np.asarray(a, dtype=np.float64)
            bf = np.asarray(b, dtype=np.float64)
            detail = [(tuple(i), af[tuple(i)], bf[tuple(i)]) for i in idx]
            raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; first {detail}")
    return check
