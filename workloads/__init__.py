"""Seeded synthetic inputs for the fused-MoE layer.

This module only draws random numbers and stores them in their storage
dtypes (bf16 bit patterns, fp8 E4M3 codes, float32, int32).  It holds none of
the layer's arithmetic -- no routing, quantiser, GEMM or reduction -- so the
CPU oracle and the HIP path can both consume its output without sharing any
of the method.

Every tensor has its own ``torch.Generator`` seeded ``1000*config + index``
(index: logits 1, x 2, W13 3, W2 4, shared W13 5, shared W2 6, residual 7,
gamma 8, hot-expert choice 9, finalize expert rows 10, finalize weight
logits 11, finalize ids 12, batched-format rows 13, batched-format counts
14).  Large weights may be drawn on the GPU with a
CUDA generator (same seeds); the CPU oracle then reads a host copy of the
very same stored values.
"""

from .configs import CONFIGS, PARITY_CASES, WorkloadSpec, FinalizeSpec  # noqa: F401
from .generate import (  # noqa: F401
    make_layer_inputs,
    make_finalize_inputs,
    make_batched_inputs,
    to_numpy_bits,
    hot_expert_tokens,
)
