"""ls_mi355: fused memory-bound non-GEMM Transformer operators for MI355X.

The operators are hand-written HIP kernels for gfx950 in ``csrc/``, built into
``libls_mi355.so`` behind the C ABI of ``include/ls_mi355.h``.  This package
is a thin binding: ``ops`` passes torch tensors' device pointers and the
current stream to the library, ``workspace`` links parameters into the
contiguous fp16 workspace of the single-launch Adam trainer.

The library is loaded lazily on first use and there is no host fallback.
"""

from ._lib import LsError, dropout_decision_bits, last_dispatch, load, version  # noqa: F401

__all__ = ["LsError", "dropout_decision_bits", "last_dispatch", "load", "version", "ops", "workspace"]


def __getattr__(name):
    if name in ("ops", "workspace", "build"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
