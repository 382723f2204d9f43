"""ctypes loader for libls_mi355.so and the declarations of its C ABI.

The library is built in-tree by ``python -m non_gemm_amd.build``.  There is no
fallback: if the shared object is missing, loading fails loudly.
"""

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libls_mi355.so")

_lock = threading.Lock()
_lib = None

c_void_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_u64 = ctypes.c_uint64
c_f32 = ctypes.c_float
c_int = ctypes.c_int
c_size = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/ls_mi355.h
SIGNATURES = {
    "ls_bias_dropout_residual": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64,
                                         c_f32, c_u64, c_u64, c_void_p]),
    "ls_bias_relu_dropout": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32, c_u64,
                                     c_u64, c_void_p]),
    "ls_elementwise_bwd_workspace_bytes": (c_size, [c_i64, c_i64]),
    "ls_bias_dropout_residual_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32, c_u64,
                                             c_u64, c_void_p, c_size, c_void_p]),
    "ls_bias_relu_dropout_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32,
                                         c_void_p, c_size, c_void_p]),
    "ls_bias_qkv_split": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p]),
    "ls_bias_qkv_split_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p,
                                      c_size, c_void_p]),
    "ls_cross_entropy_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32,
                                     ctypes.c_int32, c_void_p]),
    "ls_cross_entropy_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32,
                                     ctypes.c_int32, c_f32, c_void_p]),
    "ls_beam_topk_workspace_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "ls_beam_topk": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p,
                             c_size, c_void_p]),
    "ls_layernorm_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_i64, c_i64, c_f32, c_void_p]),
    "ls_bias_dropout_residual_layernorm": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                   c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_f32, c_u64,
                                                   c_u64, c_f32, c_void_p]),
    "ls_layernorm_bwd_workspace_bytes": (c_size, [c_i64, c_i64]),
    "ls_layernorm_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_size, c_void_p]),
    "ls_layernorm_bwd_noalloc_max_bytes": (c_size, []),
    "ls_layernorm_bwd_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_i64, c_i64, c_void_p]),
    "ls_layernorm_bwd_input": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64,
                                       c_void_p, c_size, c_void_p]),
    "ls_layernorm_bwd_params": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_void_p, c_size, c_void_p]),
    "ls_layernorm_bwd_params_batched": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                                c_void_p]),
    "ls_softmax_fwd": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_void_p, c_int,
                               c_void_p]),
    "ls_softmax_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p]),
    "ls_embedding_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64,
                                 c_i64, c_i64, c_f32, c_f32, c_u64, c_u64, c_void_p]),
    "ls_embedding_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64, c_f32,
                                 c_f32, c_u64, c_u64, c_int, c_void_p]),
    "ls_adam_workspace_step": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_i64, c_f32,
                                       c_f32, c_f32, c_f32, c_f32, c_i64, c_f32, c_int, c_void_p]),
    "ls_dropout_mask": (c_int, [c_void_p, c_i64, c_f32, c_u64, c_u64, c_void_p]),
    "ls_probe_copy": (c_int, [c_void_p, c_void_p, c_i64, c_void_p]),
    "ls_probe_read": (c_int, [c_void_p, c_void_p, c_i64, c_void_p]),
    "ls_time_next_launch": (c_int, [c_void_p, c_void_p]),
    "ls_time_armed": (c_int, []),
    "ls_dropout_decision_bits": (c_int, []),
    "ls_status_string": (ctypes.c_char_p, [c_int]),
    "ls_last_error": (ctypes.c_char_p, []),
    "ls_last_dispatch": (ctypes.c_char_p, []),
    "ls_version": (ctypes.c_char_p, []),
}


class LsError(RuntimeError):
    """A non-zero ls_status returned by the library."""

    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} failed with status {status} ({detail})")


def load(path=LIB_PATH):
    """Load the shared library once and declare every entry point."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m non_gemm_amd.build`")
        # torch's HIP runtime must be the one the library binds to (same
        # SONAME), so torch is imported before the library is opened.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(fn_name, status):
    if status != 0:
        lib = load()
        text = lib.ls_status_string(status).decode()
        detail = lib.ls_last_error().decode()
        raise LsError(fn_name, status, f"{text}: {detail}")


def last_dispatch():
    return load().ls_last_dispatch().decode()


def dropout_decision_bits():
    return int(load().ls_dropout_decision_bits())


def version():
    return load().ls_version().decode()
