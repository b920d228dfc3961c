"""GPU: the whole layer as one graph launch (moe_forward_graph_*).

The graph replays moe_forward's kernels on the buffers it was captured
with, so every replay must equal an eager moe_forward on the same inputs
bit for bit (the kernels are deterministic: align has no order-dependent
atomics, split-K partials are summed in split order).  Each case replays
the graph several times with new inputs written in place, with eager work
and host synchronisations between the replays, and checks every replay.
The last replay is also checked against the oracle, to the same bar as
the eager forward."""

import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import PARITY_CASES, make_layer_inputs, to_numpy_bits
from helpers import check_tolerance, f64_of_bf16, f64_of_fp8, output_allowance

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("decode_split_mini", "decode_split_fp8_mini", "fp8_token_mini", "fp8_tensor_mini",
         "finalize_fused_mini", "fp8_out_mini", "llama4_mini", "gelu_mini")
CASES = [s for s in PARITY_CASES if s.name in NAMES]


def _moe():
    import mixture_experts_layer_routing_amd as moe
    return moe


def _weights(moe, d, quant):
    return moe.make_weights(*(d.get(k) for k in ("w13", "w2", "w13_scale", "w2_scale", "shared_w13",
                                                 "shared_w2", "shared_w13_scale", "shared_w2_scale")),
                            quant=None if quant == "none" else quant)


def _eager(moe, spec, w, x, logits, residual, gamma):
    out, scale, _ = moe.moe_forward(x, logits, w, spec.top_k, spec.scoring, spec.renormalize,
                                    spec.apply_router_weight_on_input, spec.activation, 0, residual,
                                    gamma, spec.eps, spec.out_quant)
    return out, scale


def test_graph_cases_present():
    assert len(CASES) == len(NAMES)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_graph_replays_match_eager(spec):
    print(f"[case] graph {spec.name}", file=sys.stderr, flush=True)
    moe = _moe()
    d = {k: v.to(DEV) for k, v in make_layer_inputs(spec).items()}
    w = _weights(moe, d, spec.quant)
    # the tensors the graph is bound to
    x = d["x"].clone()
    logits = d["logits"].clone()
    residual = d.get("residual")
    gamma = d.get("gamma")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = moe.ForwardGraph(x, logits, w, spec.top_k, spec.scoring, spec.renormalize,
                             spec.apply_router_weight_on_input, spec.activation, 0, residual, gamma,
                             spec.eps, spec.out_quant)
    torch.cuda.synchronize()
    try:
        for i in range(4):
            # new inputs for replay i: scaled activations, token-rotated logits
            xi = (d["x"].float() * (0.5 + 0.5 * i)).to(torch.bfloat16)
            li = torch.roll(d["logits"], shifts=i, dims=0) * (1.0 + 0.25 * i)
            want, want_s = _eager(moe, spec, w, xi, li, residual, gamma)   # eager work in between
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                x.copy_(xi)
                logits.copy_(li)
                out, out_s = g.launch(s)
            s.synchronize()
            np.testing.assert_array_equal(to_numpy_bits(out), to_numpy_bits(want),
                                          err_msg=f"{spec.name} replay {i}")
            if out_s is not None:
                np.testing.assert_array_equal(out_s.cpu().numpy(), want_s.cpu().numpy())
            # a second launch with no input change gives the same bits again
            with torch.cuda.stream(s):
                again, _ = g.launch(s)
            s.synchronize()
            np.testing.assert_array_equal(to_numpy_bits(again), to_numpy_bits(want))
        _check_against_oracle(spec, d, xi, li, out.clone(), None if out_s is None else out_s.clone())
    finally:
        g.close()


def test_graph_on_default_stream_is_rejected():
    moe = _moe()
    spec = CASES[0]
    d = {k: v.to(DEV) for k, v in make_layer_inputs(spec).items()}
    w = _weights(moe, d, spec.quant)
    with pytest.raises(ValueError):
        with torch.cuda.stream(torch.cuda.default_stream()):
            moe.ForwardGraph(d["x"], d["logits"], w, spec.top_k)


def _check_against_oracle(spec, d, x, logits, out, out_s):
    hw = {k: to_numpy_bits(d[k]) for k in d if k.startswith(("w13", "w2", "shared"))}
    gamma = to_numpy_bits(d.get("gamma"))
    refs = {mode: oracle.forward(to_numpy_bits(x), logits.cpu().numpy(), hw, spec.top_k,
                                 spec.scoring, spec.renormalize, 16,
                                 spec.apply_router_weight_on_input, spec.quant, spec.activation,
                                 mode, to_numpy_bits(d.get("residual")), gamma, spec.eps,
                                 spec.out_quant)
            for mode in ("exact", "mirrored")}
    if spec.out_quant == "fp8":
        got = f64_of_fp8(out, out_s)
        ref = {m: f64_of_fp8(r["output"], r["output_scale"]) for m, r in refs.items()}
    else:
        got = f64_of_bf16(out)
        ref = {m: f64_of_bf16(r["output"]) for m, r in refs.items()}
    fp8 = spec.quant.startswith("fp8") or spec.out_quant == "fp8"
    d_now = dict(d, x=x)
    allowance, slack = output_allowance(spec, refs["mirrored"], d_now, hw)
    check_tolerance(got, ref["exact"], ref["mirrored"], "fp8" if fp8 else "bf16",
                    f"graph {spec.name} vs oracle", allowance=allowance, maxnorm_slack=slack)
