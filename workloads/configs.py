"""Workload shapes and value distributions.

The five measured configurations (tiny, Mixtral-shaped bf16, DeepSeek-V3-
shaped fp8, Llama-4-shaped top-1 with the router weight on the input, and
the memory-bound finalize fusion at hidden 7168) and the reduced parity cases
that keep the same structure at sizes the CPU oracle finishes in seconds
while still spanning several tiles and a ragged tail.
"""

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    config: int                 # seed base = 1000 * config
    T: int
    H: int
    I: int
    E: int
    top_k: int
    scoring: str = "softmax"    # "softmax" | "sigmoid"
    renormalize: bool = True
    quant: str = "none"         # "none" | "fp8" (G(128) acts) | "fp8_token" | "fp8_tensor"
                                # (fp8: 128x128 weight blocks)
    activation: str = "silu"    # "silu" (SiLU-mul) | "silu_no_mul" | "gelu" | "gelu_no_mul"
    apply_router_weight_on_input: bool = False
    shared_I: int = 0           # 0 = no shared expert
    logit_std: float = 1.0
    hot_experts: int = 0        # number of hot experts ...
    hot_fraction: float = 0.0   # ... and the fraction of tokens forced onto them
    hot_boost: float = 8.0      # logit added to the hot experts for those tokens
    residual: bool = False
    rmsnorm: bool = False
    eps: float = 1e-6
    out_quant: str = "none"

    def with_T(self, T):
        return replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


@dataclass(frozen=True)
class FinalizeSpec:
    name: str
    config: int
    T: int
    top_k: int = 4
    H: int = 7168
    shared: bool = True
    residual: bool = True
    rmsnorm: bool = True
    eps: float = 1e-6
    out_quant: str = "none"
    apply_router_weight_on_input: bool = False

    def with_T(self, T):
        return replace(self, T=T, name=f"{self.name.split('@')[0]}@T{T}")


TINY = WorkloadSpec("tiny", 1, T=16, H=128, I=64, E=8, top_k=2)
MIXTRAL = WorkloadSpec("mixtral", 2, T=4096, H=4096, I=14336, E=8, top_k=2, logit_std=2.0)
DEEPSEEK = WorkloadSpec("deepseek_v3", 3, T=8192, H=7168, I=2048, E=256, top_k=8,
                        scoring="sigmoid", quant="fp8", shared_I=2048,
                        hot_experts=4, hot_fraction=0.05)
LLAMA4 = WorkloadSpec("llama4", 4, T=2048, H=5120, I=8192, E=16, top_k=1,
                      renormalize=False, apply_router_weight_on_input=True, shared_I=8192)
FINALIZE = FinalizeSpec("finalize", 5, T=4096)

CONFIGS = {
    "tiny": [TINY],
    "mixtral": [MIXTRAL.with_T(t) for t in (1, 32, 512, 4096)],
    "deepseek_v3": [DEEPSEEK.with_T(t) for t in (64, 1024, 8192)],
    "llama4": [LLAMA4.with_T(t) for t in (128, 2048)]
              + [replace(LLAMA4.with_T(t), activation="silu_no_mul",
                         name=f"llama4_silu_no_mul@T{t}") for t in (128, 2048)],
    "finalize": [FINALIZE.with_T(t) for t in (128, 512, 4096, 16384)]
                + [replace(FINALIZE.with_T(t), out_quant="fp8", name=f"finalize_fp8@T{t}")
                   for t in (128, 512, 4096, 16384)],
}

# Reduced shapes with the same structure (routing rule, quant path, top-1 +
# weight on input, shared expert, hot experts), small enough for the oracle
# to finish in seconds, each spanning several M/N/K tiles with a ragged tail.
PARITY_CASES = [
    TINY,
    WorkloadSpec("mixtral_mini", 2, T=301, H=512, I=384, E=8, top_k=2, logit_std=2.0),
    WorkloadSpec("deepseek_mini", 3, T=203, H=768, I=256, E=32, top_k=8, scoring="sigmoid",
                 quant="fp8", shared_I=256, hot_experts=4, hot_fraction=0.05),
    WorkloadSpec("llama4_mini", 4, T=157, H=640, I=384, E=16, top_k=1, renormalize=False,
                 apply_router_weight_on_input=True, shared_I=512),
    WorkloadSpec("llama4_mini_silu_no_mul", 4, T=157, H=640, I=384, E=16, top_k=1,
                 renormalize=False, apply_router_weight_on_input=True, shared_I=512,
                 activation="silu_no_mul"),
    WorkloadSpec("finalize_fused_mini", 5, T=97, H=384, I=256, E=16, top_k=4,
                 shared_I=256, residual=True, rmsnorm=True),
    WorkloadSpec("fp8_out_mini", 3, T=77, H=512, I=256, E=16, top_k=4, scoring="sigmoid",
                 quant="fp8", residual=True, rmsnorm=True, out_quant="fp8"),
    # Decode-sized batches with K long enough that the GEMMs split K (a few
    # expert blocks cannot fill the GPU): bf16 SiLU-mul with a shared expert,
    # fp8, and top-1 weight-on-input silu_no_mul.
    WorkloadSpec("decode_split_mini", 6, T=5, H=2048, I=2048, E=4, top_k=2, shared_I=2048),
    WorkloadSpec("decode_split_fp8_mini", 7, T=3, H=2048, I=2048, E=16, top_k=4,
                 scoring="sigmoid", quant="fp8", shared_I=1024),
    WorkloadSpec("decode_split_no_mul_mini", 8, T=4, H=2048, I=2048, E=16, top_k=1,
                 renormalize=False, apply_router_weight_on_input=True, shared_I=2048,
                 activation="silu_no_mul"),
    # the GELU activations of the fused-experts table: gated bf16 with a
    # shared expert, ungated fp8 top-1 with the weight on the input
    WorkloadSpec("gelu_mini", 9, T=131, H=384, I=256, E=8, top_k=2, shared_I=256,
                 activation="gelu"),
    WorkloadSpec("gelu_no_mul_fp8_mini", 10, T=93, H=512, I=256, E=16, top_k=1,
                 renormalize=False, apply_router_weight_on_input=True, quant="fp8",
                 activation="gelu_no_mul"),
    # the per-token ("A") and per-tensor ("T") activation formats
    WorkloadSpec("fp8_token_mini", 16, T=117, H=768, I=256, E=32, top_k=8, scoring="sigmoid",
                 quant="fp8_token", shared_I=256, hot_experts=4, hot_fraction=0.05),
    WorkloadSpec("fp8_tensor_mini", 17, T=89, H=512, I=384, E=16, top_k=1, renormalize=False,
                 apply_router_weight_on_input=True, quant="fp8_tensor", shared_I=256),
    # enough tokens for the shared expert's 256-row dense tiles (ragged: 1100 = 4*256 + 76)
    WorkloadSpec("shared_dense_mini", 18, T=1100, H=512, I=256, E=8, top_k=2, shared_I=512,
                 residual=True, rmsnorm=True),
]
