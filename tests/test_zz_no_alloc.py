"""moe_forward_noalloc: the forward on the library's fixed per-GPU scratch.

GPU: through the C ABI, two calls in a row (the second on fewer tokens),
each bit-identical to moe_forward with a caller workspace on the same
inputs (the same kernels run), and within the parity bar of the oracle.
CPU: sizes beyond the scratch are refused before anything touches a GPU."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import PARITY_CASES, make_layer_inputs, to_numpy_bits
from helpers import check_tolerance, f64_of_bf16

CASES = {s.name: s for s in PARITY_CASES}


def _moe():
    import mixture_experts_layer_routing_amd as moe
    return moe


def _weights(moe, d, quant):
    return moe.make_weights(*(d.get(k) for k in ("w13", "w2", "w13_scale", "w2_scale", "shared_w13",
                                                 "shared_w2", "shared_w13_scale", "shared_w2_scale")),
                            quant=None if quant == "none" else quant)


def _call(moe, spec, dd, w, T):
    x, lg = dd["x"][:T].contiguous(), dd["logits"][:T].contiguous()
    res = dd["residual"][:T].contiguous() if dd.get("residual") is not None else None
    args = (x, lg, w, spec.top_k, spec.scoring, spec.renormalize,
            spec.apply_router_weight_on_input, spec.activation, 0, res, dd.get("gamma"), spec.eps,
            spec.out_quant)
    a, a_s = moe.moe_forward_noalloc(*args)
    b, b_s, _ = moe.moe_forward(*args)
    torch.cuda.synchronize()
    return a, a_s, b, b_s


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["mixtral_mini", "deepseek_mini", "llama4_mini",
                                  "finalize_fused_mini", "fp8_out_mini"])
def test_noalloc_forward_matches_forward_twice(name):
    spec = CASES[name]
    print(f"[case] noalloc {name}", file=sys.stderr, flush=True)
    moe = _moe()
    d = make_layer_inputs(spec)
    dd = {k: v.to("cuda") for k, v in d.items()}
    w = _weights(moe, dd, spec.quant)
    for T in (spec.T, max(1, spec.T // 3)):       # the second call on fewer tokens
        a, a_s, b, b_s = _call(moe, spec, dd, w, T)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} T={T}"
        if a_s is not None:
            assert torch.equal(a_s, b_s)
    # the last call against the oracle (bf16 outputs), to the parity bar
    if spec.out_quant == "none":
        hw = {k: to_numpy_bits(d[k]) for k in d if k.startswith(("w13", "w2", "shared_w"))}
        res = to_numpy_bits(d["residual"][:T]) if d.get("residual") is not None else None
        ref = oracle.forward(to_numpy_bits(d["x"][:T]), d["logits"][:T].numpy(), hw, spec.top_k,
                             spec.scoring, spec.renormalize, 16,
                             spec.apply_router_weight_on_input, spec.quant, spec.activation,
                             "mirrored", res, to_numpy_bits(d.get("gamma")), spec.eps)
        path = "fp8" if spec.quant.startswith("fp8") else "bf16"
        check_tolerance(f64_of_bf16(a), None, f64_of_bf16(ref["output"]), path, f"noalloc {name}",
                        elementwise=False)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    """Llama-4 shapes at T = 2048 need far more than 64 MiB: refused with
    MOE_ERR_WORKSPACE before any device call (the pointers are fake and the
    library never dereferences them)."""
    moe = _moe()
    L = moe.binding.lib()
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 16, 8192, 0, 8192
    w.w13 = w.w2 = w.shared_w13 = w.shared_w2 = 16
    need = L.moe_forward_workspace_bytes(2048, 5120, 1, ctypes.byref(w), 0, 0, 1)
    assert need > moe.binding.NOALLOC_SCRATCH_BYTES
    st = L.moe_forward_noalloc(16, 16, 2048, 5120, 1, 0, 0, 1, ctypes.byref(w), 0, 0, None, None,
                               1e-6, 0, 16, None, None, None)
    assert st == moe.binding.MOE_ERR_WORKSPACE
    assert "scratch" in moe.last_error()


def test_noalloc_invalid_arguments_are_reported_as_by_forward():
    moe = _moe()
    L = moe.binding.lib()
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 128, 0, 0
    w.w13 = w.w2 = 16
    # weight on the input with top_k 2: the pages' assert, before any launch
    st = L.moe_forward_noalloc(16, 16, 4, 256, 2, 0, 1, 1, ctypes.byref(w), 0, 0, None, None, 1e-6,
                               0, 16, None, None, None)
    assert st == moe.binding.MOE_ERR_INVALID_ARG
