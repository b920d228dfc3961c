"""The oracle against hand-worked examples (tests/golden/worked_examples.json)."""

import json
import os

import numpy as np

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _bf16_bits(v):
    return oracle.f64_to_bf16_bits(np.asarray(v, dtype=np.float64))


def test_golden_route():
    for key in ("route_softmax_renorm", "route_sigmoid_ties"):
        g = GOLD[key]
        ids, w = oracle.route(np.array(g["logits"], np.float32), g["top_k"], g["scoring"], g["renormalize"])
        assert ids.tolist() == g["ids"]
        np.testing.assert_allclose(w, g["weights"], rtol=0, atol=g["weight_atol"])


def test_golden_align():
    g = GOLD["align_blocks"]
    out = oracle.align(np.array(g["topk_ids"]), g["E"], g["block_m"])
    for name in ("expert_counts", "expert_offsets", "sorted_token_ids", "block_expert_ids"):
        assert out[name].tolist() == g[name], name
    assert int(out["num_tokens_post_padded"][0]) == g["num_tokens_post_padded"]


def test_golden_prepare_constant_groups():
    g = GOLD["prepare_fp8_constant_group"]
    x = np.concatenate([np.full(128, v) for v in g["values"]])[None, :]
    q, s = oracle.prepare(_bf16_bits(x), None, False, "fp8")
    assert q[0, 0] == g["codes"][0] and q[0, 128] == g["codes"][1]
    assert np.all(q[0, :128] == q[0, 0]) and np.all(q[0, 128:] == q[0, 128])


def test_golden_finalize_constant_row():
    g = GOLD["finalize_rmsnorm_constant_row"]
    H = 128
    y = _bf16_bits(np.full((1, 1, H), g["y"]))
    gamma = _bf16_bits(np.ones(H))
    out, _, _ = oracle.finalize(y, np.ones((1, 1), np.float32), False, gamma=gamma, eps=1e-6)
    assert np.all(out == g["out_bits"])
    one = _bf16_bits(np.ones((1, H)))
    out, _, _ = oracle.finalize(y, np.ones((1, 1), np.float32), False, shared=one, residual=one,
                                gamma=gamma, eps=1e-6)
    assert np.all(out == g["out_bits"])


def test_golden_prepare_per_token_and_tensor():
    g = GOLD["prepare_fp8_per_token_and_tensor"]
    x = np.concatenate([np.repeat(np.array(g["rows"], np.float64)[:, i:i + 1], 128, axis=1)
                        for i in range(2)], axis=1)                       # [2, 256]
    q, s = oracle.prepare(_bf16_bits(x), None, False, "fp8_token")
    np.testing.assert_array_equal(s[:, 0], np.array(g["token_scales"], np.float32))
    assert q[:, [0, 128]].tolist() == g["token_codes"]
    assert np.all(q[:, :128] == q[:, :1]) and np.all(q[:, 128:] == q[:, 128:129])
    q, s = oracle.prepare(_bf16_bits(x), None, False, "fp8_tensor")
    assert s.shape == (1, 1) and s[0, 0] == np.float32(g["tensor_scale"])
    assert q[:, [0, 128]].tolist() == g["tensor_codes"]


def test_golden_experts_batched():
    g = GOLD["experts_batched_hand"]
    out = oracle.experts_batched(_bf16_bits(g["a"]), None, g["counts"], _bf16_bits(g["w13"]), None,
                                 _bf16_bits(g["w2"]), None, "silu")
    np.testing.assert_array_equal(out, _bf16_bits(g["out"]))
