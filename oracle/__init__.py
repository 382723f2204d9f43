"""CPU oracle for the fused non-GEMM Transformer operators.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, header, table or helper with
the HIP library under ``non_gemm_amd/``, and it imports nothing from it.

Every function takes and returns NumPy arrays.  Inputs are the exact fp16 /
int32 arrays the GPU receives; the oracle widens them to float64, computes the
plain textbook definition (two-pass LayerNorm, two-pass softmax, dense
scatter-add for the embedding gradient, Adam written out term by term) and
rounds once at each point where the GPU path stores a value (fp16 outputs with
round-to-nearest-even, fp32 statistics and moments).

Sources (cited by page title and section; no line numbers):

* [L10]  CMU 11-868 L10 digest, "Accelerating Transformer on GPU: where
  LightSeq saves its time" (quidproquo.cc) -- technique 1 (kernel fusion,
  slide 12), technique 2 (formula rewriting, slides 21-26), technique 3
  (mixed precision, slides 27-29).
* [LS2]  "LightSeq2: Accelerated Training for Transformer-based Models on
  GPUs", reading notes (arcsin2.cloud) -- sec. 2.1.1 (layer operators),
  sec. 2.1.2 (embedding forward / backward equations), sec. 2.3 (mixed
  precision trainer).
* [CS336] Stanford CS336 lecture 5 notes, "GPU" (auss.cc) -- sec. 3.2
  (mixed precision, loss scaling), sec. 6.2 (online softmax).
* [SC11] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
  1, 2, 3", SC'11 -- the Philox4x32-10 bijection.

Parity status per function is listed in each function's docstring; every
function here is pinned by at least one independent check in
``tests/test_oracle_*.py``.
"""

from . import philox  # noqa: F401
from .ops import (  # noqa: F401
    adam_workspace_step,
    bias_dropout_residual,
    bias_dropout_residual_bwd,
    bias_dropout_residual_layernorm,
    bias_qkv_split,
    bias_qkv_split_bwd,
    bias_relu_dropout,
    bias_relu_dropout_bwd,
    cross_entropy_bwd,
    cross_entropy_fwd,
    dropout_keep,
    dropout_scale,
    beam_candidates,
    embedding_bwd,
    hars_topk,
    embedding_fwd,
    layernorm_bwd,
    layernorm_fwd,
    softmax_bwd,
    softmax_fwd,
)
