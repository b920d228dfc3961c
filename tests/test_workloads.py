"""The seeded input recipes: deterministic, the stated shapes and spreads, and
the oracle runs end to end on every reduced parity case."""

import time

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PARITY_CASES, make_layer_inputs, make_finalize_inputs, to_numpy_bits
from workloads.generate import hot_expert_tokens


def test_generation_is_deterministic():
    spec = PARITY_CASES[2]
    a, b = make_layer_inputs(spec), make_layer_inputs(spec)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_spreads_follow_the_recipe():
    spec = PARITY_CASES[1]                      # bf16, logit std 2
    d = make_layer_inputs(spec)
    assert abs(d["logits"].std().item() - 2.0) < 0.15
    assert abs(d["x"].float().std().item() - 1.0) < 0.05
    assert abs(d["w13"].float().std().item() * np.sqrt(spec.H) - 1.0) < 0.05
    assert abs(d["w2"].float().std().item() * np.sqrt(spec.I) - 1.0) < 0.05
    f8 = make_layer_inputs(PARITY_CASES[2])     # fp8 codes x block scales
    deq = oracle.moe.dequant_weight(to_numpy_bits(f8["w13"][0]), to_numpy_bits(f8["w13_scale"][0]))
    assert 0.8 < deq.std() * np.sqrt(PARITY_CASES[2].H) < 1.2


def test_hot_experts_land_in_every_forced_tokens_top_k():
    spec = CONFIGS["deepseek_v3"][0]            # T = 64, E = 256, k = 8
    d = make_layer_inputs(spec, weights=False)
    ids, _ = oracle.route(d["logits"].numpy(), spec.top_k, spec.scoring, spec.renormalize)
    hot, toks = hot_expert_tokens(spec)
    assert toks.numel() == round(0.05 * spec.T)
    for t in toks.tolist():
        assert set(hot.tolist()) <= set(ids[t].tolist())


def test_finalize_inputs_recipe():
    spec = CONFIGS["finalize"][0]
    d = make_finalize_inputs(spec)
    assert d["fused_expert_output"].shape == (spec.T, 4, 7168)
    np.testing.assert_allclose(d["topk_weights"].sum(1).numpy(), 1.0, atol=1e-6)
    ids = d["topk_ids"]
    assert all(len(set(r)) == 4 for r in ids.tolist()) and ids.max() < 256
    g = d["gamma"].float()
    assert g.min() >= 0.5 and g.max() <= 1.5


@pytest.mark.parametrize("spec", PARITY_CASES, ids=lambda s: s.name)
def test_oracle_runs_on_reduced_cases(spec):
    d = make_layer_inputs(spec)
    w = {k: to_numpy_bits(v) for k, v in d.items() if k.startswith(("w13", "w2", "shared"))}
    t0 = time.time()
    out = oracle.forward(to_numpy_bits(d["x"]), d["logits"].numpy(), w, spec.top_k, spec.scoring,
                         spec.renormalize, 16, spec.apply_router_weight_on_input, spec.quant,
                         spec.activation, "mirrored", to_numpy_bits(d.get("residual")),
                         to_numpy_bits(d.get("gamma")), spec.eps, spec.out_quant)
    assert time.time() - t0 < 30
    assert out["output"].shape == (spec.T, spec.H)
    assert np.isfinite(oracle.bf16_bits_to_f64(out["fused_expert_output"])).all()
