"""The per-element parity check itself: it admits exactly the one-step bf16
rounding flips of the expert rows that two correct implementations may
disagree on, and rejects plausible mistakes (a dropped routed slot, a
doubled router weight, a wrong expert row)."""

import numpy as np
import pytest

import oracle
from helpers import check_tolerance, finalize_flip_allowance, f64_of_bf16
from workloads import PARITY_CASES, make_layer_inputs, to_numpy_bits

CASES = [s for s in PARITY_CASES if s.quant == "none" and s.out_quant == "none"]


def _forward(spec):
    d = make_layer_inputs(spec)
    hw = {k: to_numpy_bits(v) for k, v in d.items() if k.startswith(("w", "shared"))}
    ref = oracle.forward(to_numpy_bits(d["x"]), d["logits"].numpy(), hw, spec.top_k, spec.scoring,
                         spec.renormalize, 16, spec.apply_router_weight_on_input, spec.quant,
                         spec.activation, "mirrored", to_numpy_bits(d.get("residual")),
                         to_numpy_bits(d.get("gamma")), spec.eps, spec.out_quant)
    return d, ref


def _refinalize(spec, d, ref, feo, tw=None):
    out, _, _ = oracle.finalize(feo, ref["topk_weights"] if tw is None else tw,
                                spec.apply_router_weight_on_input, ref["shared_out"],
                                to_numpy_bits(d.get("residual")), to_numpy_bits(d.get("gamma")),
                                spec.eps, "none")
    return f64_of_bf16(out)


def _check(spec, d, ref, got):
    exact = f64_of_bf16(ref["output"])
    return check_tolerance(got, exact, exact, "bf16", spec.name,
                           allowance=finalize_flip_allowance(ref, to_numpy_bits(d.get("gamma")),
                                                             spec.apply_router_weight_on_input))


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_one_step_flips_of_expert_rows_pass(spec):
    d, ref = _forward(spec)
    feo = np.array(ref["fused_expert_output"], dtype=np.uint16)
    rng = np.random.default_rng(7)
    nz = (feo & 0x7FFF) != 0
    # flip a third of the nonzero elements one bf16 step away from or toward zero
    flip = nz & (rng.random(feo.shape) < 1 / 3)
    step = np.where(rng.random(feo.shape) < 0.5, 1, -1).astype(np.int32)
    pert = np.where(flip, (feo.astype(np.int32) + step), feo.astype(np.int32)).astype(np.uint16)
    _check(spec, d, ref, _refinalize(spec, d, ref, pert))


@pytest.mark.parametrize("spec", CASES, ids=lambda s: s.name)
def test_planted_mistakes_fail(spec):
    d, ref = _forward(spec)
    feo = np.array(ref["fused_expert_output"], dtype=np.uint16)
    if spec.top_k > 1 and not spec.apply_router_weight_on_input:
        dropped = feo.copy()
        dropped[:, -1, :] = 0                      # last routed slot lost
        with pytest.raises(AssertionError):
            _check(spec, d, ref, _refinalize(spec, d, ref, dropped))
        tw = np.array(ref["topk_weights"], copy=True)
        tw[:, 0] *= 2                              # weight applied twice
        with pytest.raises(AssertionError):
            _check(spec, d, ref, _refinalize(spec, d, ref, feo, tw))
    swapped = feo.copy()
    swapped[0], swapped[-1] = feo[-1], feo[0]      # rows of two tokens exchanged
    with pytest.raises(AssertionError):
        _check(spec, d, ref, _refinalize(spec, d, ref, swapped))


def test_flip_allowance_uses_weight_one_when_the_weight_went_on_the_input():
    """With the router weight on the input, finalize adds the expert row
    with weight 1, so a one-step flip of that row moves the output by a
    whole step of the row, not by w times it."""
    spec = next(s for s in CASES if s.apply_router_weight_on_input)
    d, ref = _forward(spec)
    tok = ref["tokens"]
    y = f64_of_bf16(ref["fused_expert_output"])[tok][:, 0]
    from helpers import bf16_ulp
    allow = finalize_flip_allowance(ref, None, weight_on_input=True)
    assert np.all(allow >= bf16_ulp(y))
    w = np.asarray(ref["topk_weights"], np.float64)[tok]
    assert w.max() < 1.0          # the weighted allowance would be smaller
    assert np.any(finalize_flip_allowance(ref, None) < bf16_ulp(y))
