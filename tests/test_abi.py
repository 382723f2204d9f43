"""Host-side checks of the C ABI (CPU only: no kernel is ever launched).

The library must load, export every function include/ls_mi355.h declares,
and reject invalid arguments with the documented status before touching the
GPU.  Every call below fails validation, so no HIP work is enqueued.
"""
import ctypes
import os
import re

import pytest

from non_gemm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ls_mi355.h")

LS_OK, LS_ERR_NULL, LS_ERR_SHAPE, LS_ERR_PARAM, LS_ERR_WORKSPACE, LS_ERR_UNSUPPORTED = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ls_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    # LS_MI355_TEST_LIB: another build of the same library (the host-sanitized
    # one, run by test_abi_sanitized.py)
    other = os.environ.get("LS_MI355_TEST_LIB")
    if other:
        return _lib.load(other)
    if not os.path.exists(_lib.LIB_PATH):
        from non_gemm_amd import build
        build.build()
    return _lib.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_introspection(lib):
    assert lib.ls_dropout_decision_bits() == 16
    assert lib.ls_version().decode().startswith("ls_mi355")
    assert lib.ls_status_string(LS_ERR_WORKSPACE).decode() == "workspace too small"
    assert lib.ls_status_string(99).decode() == "unknown status"


def test_elementwise_validation(lib):
    s = None
    assert lib.ls_bias_dropout_residual(FAKE, FAKE, FAKE, FAKE, -1, 8, 0.1, 1, 0, s) == LS_ERR_SHAPE
    assert lib.ls_bias_dropout_residual(FAKE, FAKE, FAKE, FAKE, 4, 8, 1.5, 1, 0, s) == LS_ERR_PARAM
    assert lib.ls_bias_dropout_residual(FAKE, FAKE, FAKE, FAKE, 4, 8, float("nan"), 1, 0, s) == LS_ERR_PARAM
    assert lib.ls_bias_dropout_residual(FAKE, None, FAKE, FAKE, 4, 8, 0.1, 1, 0, s) == LS_ERR_NULL
    assert b"null" in lib.ls_last_error()
    assert lib.ls_bias_relu_dropout(FAKE, FAKE, None, 4, 8, 0.1, 1, 0, s) == LS_ERR_NULL
    assert lib.ls_bias_relu_dropout(FAKE, FAKE, FAKE, 4, 8, -0.1, 1, 0, s) == LS_ERR_PARAM
    # empty tensors are valid no-ops, NULL pointers allowed
    assert lib.ls_bias_relu_dropout(None, None, None, 0, 8, 0.1, 1, 0, s) == LS_OK
    assert lib.ls_last_dispatch() == b"empty"
    assert lib.ls_dropout_mask(None, 0, 0.5, 1, 0, s) == LS_OK
    assert lib.ls_dropout_mask(None, 10, 0.5, 1, 0, s) == LS_ERR_NULL
    assert lib.ls_dropout_mask(FAKE, -1, 0.5, 1, 0, s) == LS_ERR_SHAPE


def test_layernorm_validation(lib):
    s = None
    assert lib.ls_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 0.0, s) == LS_ERR_PARAM
    assert lib.ls_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 1e-5, s) == LS_ERR_SHAPE
    assert lib.ls_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8192, 1e-5, s) == LS_ERR_UNSUPPORTED
    assert lib.ls_layernorm_fwd(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 1e-5, s) == LS_ERR_NULL
    assert lib.ls_layernorm_fwd(None, None, None, None, None, None, 0, 8, 1e-5, s) == LS_OK
    # 2^31 rows and more are refused before anything is launched (32-bit row loops)
    assert lib.ls_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 31, 8, 1e-5, s) == LS_ERR_SHAPE
    assert lib.ls_layernorm_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 31, 8,
                                FAKE, 1 << 40, s) == LS_ERR_SHAPE
    need = lib.ls_layernorm_bwd_workspace_bytes(4096, 768)
    assert need == 256 + 256 * 2 * 768 * 4          # header, then at most 256 partial rows of 2H floats
    assert lib.ls_layernorm_bwd_workspace_bytes(5, 768) == 256 + 5 * 2 * 768 * 4
    assert lib.ls_layernorm_bwd_workspace_bytes(0, 768) == 0
    assert lib.ls_layernorm_bwd_workspace_bytes(10, 5000) == 0
    assert lib.ls_layernorm_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 768,
                                FAKE, need - 1, s) == LS_ERR_WORKSPACE
    assert lib.ls_layernorm_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 768,
                                None, need, s) == LS_ERR_NULL
    assert lib.ls_layernorm_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 768,
                                ctypes.c_void_p(0x1008), need, s) == LS_ERR_PARAM
    # the two halves validate the same way; nothing is launched on these paths
    assert lib.ls_layernorm_bwd_input(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, 768, FAKE, need - 1,
                                      s) == LS_ERR_WORKSPACE
    assert lib.ls_layernorm_bwd_input(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4096, 768, FAKE, need, s) == LS_ERR_NULL
    assert lib.ls_layernorm_bwd_input(None, None, None, None, None, None, 0, 768, None, 0, s) == LS_OK
    assert lib.ls_layernorm_bwd_params(FAKE, FAKE, 4096, 768, FAKE, need - 1, s) == LS_ERR_WORKSPACE
    assert lib.ls_layernorm_bwd_params(FAKE, FAKE, 4096, 768, None, need, s) == LS_ERR_NULL
    assert lib.ls_layernorm_bwd_params(None, FAKE, 0, 768, None, 0, s) == LS_ERR_NULL
    assert lib.ls_layernorm_bwd_params(FAKE, FAKE, 4096, 5000, FAKE, need, s) == LS_ERR_UNSUPPORTED
    assert lib.ls_layernorm_bwd_params(FAKE, FAKE, -1, 768, FAKE, need, s) == LS_ERR_SHAPE
    assert lib.ls_layernorm_bwd_params(FAKE, FAKE, 4096, 768, ctypes.c_void_p(0x1008), need, s) == LS_ERR_PARAM
    # rows == 0: the zero-row sums still need their outputs
    assert lib.ls_layernorm_bwd(None, None, FAKE, None, None, None, None, None, 0, 768, None, 0, s) == LS_ERR_NULL


def test_layernorm_params_batched_validation(lib):
    """The batched finalisation checks every job before launching anything;
    the error names the first failing job."""
    s = None
    need = lib.ls_layernorm_bwd_workspace_bytes(4096, 768)
    P = ctypes.c_void_p * 3
    I = ctypes.c_int64 * 3
    Z = ctypes.c_size_t * 3

    def call(n, dg, db, rows, hid, ws, nb):
        return lib.ls_layernorm_bwd_params_batched(n, P(*dg), P(*db), I(*rows), I(*hid), P(*ws), Z(*nb), s)

    ok = ([FAKE] * 3, [FAKE] * 3, [4096, 0, 5], [768, 768, 0], [FAKE, None, None], [need, 0, 0])
    assert lib.ls_layernorm_bwd_params_batched(-1, None, None, None, None, None, None, s) == LS_ERR_PARAM
    assert lib.ls_layernorm_bwd_params_batched(0, None, None, None, None, None, None, s) == LS_OK
    assert lib.ls_last_dispatch() == b"empty"
    assert lib.ls_layernorm_bwd_params_batched(1, None, None, None, None, None, None, s) == LS_ERR_NULL
    # job 2: hidden 0 is skipped (nothing to write, its pointers unread); only
    # hidden == 0 jobs: nothing launched
    assert call(3, [None] * 3, [None] * 3, [7, 0, 1], [0, 0, 0], [None] * 3, [0] * 3) == LS_OK
    assert lib.ls_last_dispatch() == b"empty"
    for job, field, bad, code in [(0, 5, need - 1, LS_ERR_WORKSPACE), (0, 4, None, LS_ERR_NULL),
                                  (1, 0, None, LS_ERR_NULL), (0, 3, 5000, LS_ERR_UNSUPPORTED),
                                  (1, 2, -1, LS_ERR_SHAPE), (0, 4, ctypes.c_void_p(0x1008), LS_ERR_PARAM),
                                  (0, 2, 1 << 31, LS_ERR_SHAPE)]:
        args = [list(a) for a in ok]
        args[field][job] = bad
        assert call(3, *args) == code, (job, field, bad)
        assert f"ls_layernorm_bwd_params_batched: job {job}:".encode() in lib.ls_last_error()


def test_softmax_validation(lib):
    s = None
    assert lib.ls_softmax_fwd(FAKE, FAKE, 2, 2, 4, -1, None, 0, s) == LS_ERR_SHAPE
    assert lib.ls_softmax_fwd(FAKE, FAKE, 1, 1, 1, 65544, None, 0, s) == LS_ERR_UNSUPPORTED
    assert lib.ls_softmax_fwd(FAKE, FAKE, 1, 1, 1, 1030, None, 0, s) == LS_ERR_UNSUPPORTED   # element-wise path limit
    assert lib.ls_softmax_fwd(None, FAKE, 1, 1, 1, 128, None, 0, s) == LS_ERR_NULL
    assert lib.ls_softmax_fwd(FAKE, FAKE, 1 << 20, 1 << 10, 1 << 10, 128, None, 0, s) == LS_ERR_SHAPE
    assert lib.ls_softmax_fwd(None, None, 0, 12, 128, 128, None, 1, s) == LS_OK
    assert lib.ls_softmax_bwd(FAKE, None, FAKE, 4, 128, s) == LS_ERR_NULL
    assert lib.ls_softmax_bwd(None, None, None, 0, 128, s) == LS_OK
    assert lib.ls_softmax_bwd(FAKE, FAKE, FAKE, 1 << 31, 128, s) == LS_ERR_SHAPE      # 32-bit row loops


def test_embedding_validation(lib):
    s = None
    assert lib.ls_embedding_fwd(FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 10, 8, 1.0, 0.1, 1, 0, s) == LS_ERR_SHAPE
    assert lib.ls_embedding_fwd(FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 10, 16, 1.0, 2.0, 1, 0, s) == LS_ERR_PARAM
    assert lib.ls_embedding_fwd(FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 10, 16, float("inf"), 0.1, 1, 0, s) == LS_ERR_PARAM
    assert lib.ls_embedding_fwd(FAKE, None, FAKE, FAKE, 2, 16, 8, 10, 16, 1.0, 0.1, 1, 0, s) == LS_ERR_NULL
    assert lib.ls_embedding_bwd(None, FAKE, FAKE, 2, 16, 8, 10, 1.0, 0.1, 1, 0, 1, s) == LS_ERR_NULL
    assert lib.ls_embedding_bwd(FAKE, FAKE, FAKE, -2, 16, 8, 10, 1.0, 0.1, 1, 0, 1, s) == LS_ERR_SHAPE
    assert lib.ls_embedding_bwd(FAKE, FAKE, FAKE, 2, 16, 8, 10, 1.0, 1.1, 1, 0, 1, s) == LS_ERR_PARAM
    assert lib.ls_embedding_bwd(None, None, None, 0, 16, 8, 0, 1.0, 0.1, 1, 0, 1, s) == LS_OK


def test_adam_validation(lib):
    s = None
    a = (FAKE, FAKE, FAKE, FAKE, 100)
    assert lib.ls_adam_workspace_step(*a, 1e-3, 0.9, 0.999, 1e-8, 0.0, 0, 1.0, 1, s) == LS_ERR_PARAM
    assert lib.ls_adam_workspace_step(*a, 1e-3, 1.0, 0.999, 1e-8, 0.0, 1, 1.0, 1, s) == LS_ERR_PARAM
    assert lib.ls_adam_workspace_step(*a, 1e-3, 0.9, 0.999, 0.0, 0.0, 1, 1.0, 1, s) == LS_ERR_PARAM
    assert lib.ls_adam_workspace_step(*a, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 0.0, 1, s) == LS_ERR_PARAM
    assert lib.ls_adam_workspace_step(*a, -1.0, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 1, s) == LS_ERR_PARAM
    assert lib.ls_adam_workspace_step(FAKE, None, FAKE, FAKE, 100, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 1, s) == LS_ERR_NULL
    assert lib.ls_adam_workspace_step(None, None, None, None, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, 1.0, 1, s) == LS_OK


def test_probe_validation(lib):
    s = None
    assert lib.ls_probe_copy(FAKE, FAKE, 24, s) == LS_ERR_SHAPE
    assert lib.ls_probe_copy(FAKE, FAKE, -16, s) == LS_ERR_SHAPE
    assert lib.ls_probe_copy(None, FAKE, 32, s) == LS_ERR_NULL
    assert lib.ls_probe_copy(ctypes.c_void_p(0x1008), FAKE, 32, s) == LS_ERR_PARAM
    assert lib.ls_probe_copy(None, None, 0, s) == LS_OK
    assert lib.ls_probe_read(None, FAKE, 1024, s) == LS_ERR_NULL
    assert lib.ls_probe_read(FAKE, FAKE, 1000, s) == LS_ERR_SHAPE
    assert lib.ls_probe_read(None, None, 0, s) == LS_OK


def test_elementwise_bwd_validation(lib):
    s = None
    need = lib.ls_elementwise_bwd_workspace_bytes(4096, 768)
    assert need > 0 and need % (768 * 4) == 0
    assert lib.ls_elementwise_bwd_workspace_bytes(0, 768) == 0
    assert lib.ls_elementwise_bwd_workspace_bytes(10, 0) == 0
    a = (FAKE, FAKE, FAKE, 4096, 768)
    assert lib.ls_bias_dropout_residual_bwd(*a, 0.1, 1, 0, FAKE, need - 1, s) == LS_ERR_WORKSPACE
    assert lib.ls_bias_dropout_residual_bwd(*a, 0.1, 1, 0, None, need, s) == LS_ERR_NULL
    assert lib.ls_bias_dropout_residual_bwd(*a, 0.1, 1, 0, ctypes.c_void_p(0x1008), need, s) == LS_ERR_PARAM
    assert lib.ls_bias_dropout_residual_bwd(*a, 1.5, 1, 0, FAKE, need, s) == LS_ERR_PARAM
    assert lib.ls_bias_dropout_residual_bwd(FAKE, None, FAKE, 4096, 768, 0.1, 1, 0, FAKE, need, s) == LS_ERR_NULL
    assert lib.ls_bias_dropout_residual_bwd(FAKE, FAKE, FAKE, -1, 768, 0.1, 1, 0, FAKE, need, s) == LS_ERR_SHAPE
    assert lib.ls_bias_dropout_residual_bwd(None, None, None, 5, 0, 0.1, 1, 0, None, 0, s) == LS_OK
    assert lib.ls_bias_relu_dropout_bwd(FAKE, FAKE, FAKE, None, 4096, 768, 0.1, FAKE, need, s) == LS_ERR_NULL
    assert lib.ls_bias_relu_dropout_bwd(FAKE, FAKE, FAKE, FAKE, 4096, 768, float("nan"), FAKE, need, s) == LS_ERR_PARAM
    assert lib.ls_bias_relu_dropout_bwd(FAKE, FAKE, FAKE, FAKE, 4096, 768, 0.1, FAKE, need - 4, s) == LS_ERR_WORKSPACE


def test_qkv_split_validation(lib):
    s = None
    assert lib.ls_bias_qkv_split(FAKE, FAKE, FAKE, -1, 128, 12, 64, s) == LS_ERR_SHAPE
    assert lib.ls_bias_qkv_split(FAKE, None, FAKE, 32, 128, 12, 64, s) == LS_ERR_NULL
    assert lib.ls_bias_qkv_split(None, None, None, 0, 128, 12, 64, s) == LS_OK
    assert lib.ls_bias_qkv_split(FAKE, FAKE, FAKE, 1 << 31, 1 << 31, 1 << 20, 1 << 20, s) == LS_ERR_SHAPE
    need = lib.ls_elementwise_bwd_workspace_bytes(4096, 2304)
    assert lib.ls_bias_qkv_split_bwd(FAKE, FAKE, FAKE, 32, 128, 12, 64, FAKE, need - 1, s) == LS_ERR_WORKSPACE
    assert lib.ls_bias_qkv_split_bwd(FAKE, None, FAKE, 32, 128, 12, 64, FAKE, need, s) == LS_ERR_NULL
    assert lib.ls_bias_qkv_split_bwd(FAKE, FAKE, None, 32, 128, 12, 64, FAKE, need, s) == LS_ERR_NULL
    assert lib.ls_bias_qkv_split_bwd(None, None, None, 32, 128, 0, 64, None, 0, s) == LS_OK


def test_cross_entropy_validation(lib):
    s = None
    assert lib.ls_cross_entropy_fwd(FAKE, FAKE, FAKE, FAKE, -1, 100, 0.1, -1, s) == LS_ERR_SHAPE
    assert lib.ls_cross_entropy_fwd(FAKE, FAKE, FAKE, FAKE, 4, 100, 1.5, -1, s) == LS_ERR_PARAM
    assert lib.ls_cross_entropy_fwd(FAKE, FAKE, FAKE, FAKE, 4, 100, float("nan"), -1, s) == LS_ERR_PARAM
    assert lib.ls_cross_entropy_fwd(FAKE, None, FAKE, FAKE, 4, 100, 0.1, -1, s) == LS_ERR_NULL
    assert lib.ls_cross_entropy_fwd(FAKE, FAKE, FAKE, FAKE, 4, 0, 0.1, -1, s) == LS_ERR_SHAPE
    assert lib.ls_cross_entropy_fwd(None, None, None, None, 0, 100, 0.1, -1, s) == LS_OK
    assert lib.ls_cross_entropy_bwd(FAKE, FAKE, FAKE, None, 4, 100, 0.1, -1, 1.0, s) == LS_ERR_NULL
    assert lib.ls_cross_entropy_bwd(FAKE, FAKE, FAKE, FAKE, 4, 100, 0.1, -1, float("inf"), s) == LS_ERR_PARAM
    assert lib.ls_cross_entropy_bwd(None, None, None, None, 0, 100, 0.1, -1, 1.0, s) == LS_OK


def test_beam_topk_validation(lib):
    s = None
    need = lib.ls_beam_topk_workspace_bytes(2, 4, 4)
    assert need == 2 * 4 * 4 * 8
    assert lib.ls_beam_topk_workspace_bytes(2, 64, 128) == 0
    w = (FAKE, need)
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, -1, 4, 100, 4, *w, s) == LS_ERR_SHAPE
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 4, 100, 401, *w, s) == LS_ERR_SHAPE
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 4, 1000, 1025, *w, s) == LS_ERR_UNSUPPORTED
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 8, 1000, 1000, *w, s) == LS_ERR_UNSUPPORTED
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 1 << 16, 1 << 16, 4, *w, s) == LS_ERR_SHAPE
    assert lib.ls_beam_topk(FAKE, None, FAKE, None, 2, 4, 100, 4, *w, s) == LS_ERR_NULL
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 4, 100, 4, FAKE, need - 8, s) == LS_ERR_WORKSPACE
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 4, 100, 4, None, need, s) == LS_ERR_NULL
    assert lib.ls_beam_topk(FAKE, FAKE, FAKE, None, 2, 4, 100, 4, ctypes.c_void_p(0x1004), need, s) == LS_ERR_PARAM
    assert lib.ls_beam_topk(None, None, None, None, 0, 4, 100, 4, None, 0, s) == LS_OK


def test_time_next_launch_validation(lib):
    assert lib.ls_time_next_launch(None, FAKE) == LS_ERR_NULL
    assert lib.ls_time_next_launch(FAKE, None) == LS_ERR_NULL
    assert b"null event" in lib.ls_last_error()


def test_timing_events_last_one_operator_call(lib):
    """Armed events belong to the next operator call, whatever it does: a
    call rejected before launching, or one with nothing to launch, disarms
    them, so they never attach to a later, unrelated kernel."""
    s = None
    assert lib.ls_time_next_launch(FAKE, FAKE) == LS_OK and lib.ls_time_armed() == 1
    lib.ls_layernorm_bwd_workspace_bytes(8, 8)                     # a size query is not an operator call
    assert lib.ls_time_armed() == 1
    assert lib.ls_layernorm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 0.0, s) == LS_ERR_PARAM
    assert lib.ls_time_armed() == 0
    assert lib.ls_time_next_launch(FAKE, FAKE) == LS_OK
    assert lib.ls_bias_relu_dropout(None, None, None, 0, 8, 0.1, 1, 0, s) == LS_OK      # empty: no launch
    assert lib.ls_time_armed() == 0
    assert lib.ls_time_next_launch(FAKE, FAKE) == LS_OK
    assert lib.ls_softmax_bwd(FAKE, None, FAKE, 4, 128, s) == LS_ERR_NULL               # not a hooked operator
    assert lib.ls_time_armed() == 0
    assert lib.ls_time_next_launch(None, FAKE) == LS_ERR_NULL and lib.ls_time_armed() == 0
