"""CPU oracle for the no-DP/EP fused-MoE layer (route -> prepare -> align ->
experts -> finalize).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
reference the HIP kernels are checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it.  The product path (``mixture_experts_layer_routing_amd``) never
imports, links or runs anything in here, and nothing in here imports the
product path: the two share no kernels, headers, helpers, tables or codecs.

Arithmetic is numpy float64 unless a step's result is a code decided by
floating point (an fp8 quantised code, a top-k choice): such decisions are
taken in float32, the precision the kernels take them in, so that only one
answer is correct.  Values whose storage type the pages fix (bf16 activations
and expert outputs, fp8 prepare output) are rounded to that type where the
pages put the boundary.

Sources ("the pages"):
  * "Fused MoE Kernel Features" (vLLM design doc, Korean rendering) -- the
    modular prepare/finalize contract, activation formats, quant formats
    G(128)/A/T, apply-router-weight-on-input for top-1, activation names.
  * "[vLLM] MoE Oracle & Prepare/Finalize" -- the no-DP/EP prepare/finalize
    code: prepare multiplies the top-1 weight into the input then quantises;
    finalize hands the expert outputs to a weight-and-reduce step.
  * "[flashinfer] MoE Finalize + AllReduce fusion ... shared-expert two-shot
    program" -- finalize = routing-scale-weighted top-k sum plus optional
    shared-expert row, residual add, RMSNorm at hidden 7168.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against library routines (torch CPU casts, float64 softmax/sigmoid, matmul,
``F.rms_norm``), brute force, closed forms and invariants.  The one reading
with no independent pin is the precision of the experts' intermediate
activation (bf16, or fp8 G(128) along I on the fp8 path): "parity unpinned"
for ``mode="mirrored"`` beyond what the tolerance bound covers.
"""

from .codecs import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    e4m3_decode,
    e4m3_encode_sat,
    E4M3_MAX,
)
from .moe import (  # noqa: F401
    route,
    prepare,
    quantize_g128,
    quantize_token,
    quantize_tensor,
    dequant_g128,
    dequant_scaled,
    align,
    align_capacity,
    experts,
    experts_batched,
    finalize,
    forward,
    silu,
    gelu,
)
