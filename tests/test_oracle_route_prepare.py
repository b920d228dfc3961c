"""Pins of the oracle's routing and prepare steps: brute force, library
routines (torch float64 softmax/sigmoid, torch CPU bf16 multiply and fp8
cast), closed forms and invariants."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs


# ----------------------------------------------------------------- route
def _brute_topk(row, k):
    keyed = sorted(((-float(v), e) for e, v in enumerate(row)))
    return [e for _, e in keyed[:k]]


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (33, 16, 1), (25, 256, 8), (7, 5, 5)])
def test_route_ids_brute_force_with_frequent_ties(T, E, k):
    rng = np.random.default_rng(T * E + k)
    # logits from a tiny set of values so ties are common
    logits = rng.integers(-3, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
    ids, _ = oracle.route(logits, k, "softmax", True)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(logits[t], k)


@pytest.mark.parametrize("scoring,renorm", [("softmax", True), ("softmax", False),
                                            ("sigmoid", True), ("sigmoid", False)])
def test_route_weights_match_torch_float64(scoring, renorm):
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 2, size=(64, 32)).astype(np.float32)
    ids, w = oracle.route(logits, 6, scoring, renorm)
    lt = torch.from_numpy(logits).double()
    p = torch.softmax(lt, dim=1) if scoring == "softmax" else torch.sigmoid(lt)
    ref = torch.gather(p, 1, torch.from_numpy(ids.astype(np.int64)))
    if renorm:
        ref = ref / ref.sum(dim=1, keepdim=True)
    np.testing.assert_allclose(w, ref.float().numpy(), rtol=0, atol=1e-7)
    # torch's own top-k picks the same set of experts (distinct logits here)
    tk = torch.topk(lt, 6, dim=1).indices.numpy()
    np.testing.assert_array_equal(ids, tk)


def test_route_invariants():
    rng = np.random.default_rng(6)
    logits = rng.normal(size=(100, 16)).astype(np.float32)
    ids, w = oracle.route(logits, 4, "softmax", True)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == 4 for r in ids.tolist())
    assert ids.min() >= 0 and ids.max() < 16
    picked = np.take_along_axis(logits, ids.astype(np.int64), 1)
    assert np.all(np.diff(picked, axis=1) <= 0)          # non-increasing along slots
    _, w_all = oracle.route(logits, 16, "softmax", False)
    np.testing.assert_allclose(w_all.sum(1), 1.0, atol=1e-6)   # k = E: all of softmax
    _, w1 = oracle.route(logits, 1, "softmax", True)
    assert np.all(w1 == 1.0)                                    # k = 1 renormalised
    _, wn = oracle.route(logits, 4, "softmax", False)
    assert np.all(wn.sum(1) <= 1.0 + 1e-6)


def test_route_equal_logits_special_case():
    logits = np.full((3, 10), 0.25, dtype=np.float32)
    ids, w = oracle.route(logits, 4, "softmax", True)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    np.testing.assert_allclose(w, 0.25, atol=1e-7)
    ids, w = oracle.route(logits, 4, "sigmoid", True)
    np.testing.assert_allclose(w, 0.25, atol=1e-7)


def test_route_negative_zero_ties_with_zero():
    logits = np.array([[-0.0, 0.0, -1.0]], dtype=np.float32)
    ids, _ = oracle.route(logits, 2, "softmax", True)
    assert ids.tolist() == [[0, 1]]


# --------------------------------------------------------------- prepare
def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_prepare_passthrough_without_quant_or_flag():
    rng = np.random.default_rng(1)
    x = _bits(_bf16(rng.normal(size=(5, 256))))
    a, s = oracle.prepare(x, None, False, "none")
    assert s is None and np.array_equal(a, x)


def test_prepare_weight_on_input_matches_torch_bf16_multiply():
    rng = np.random.default_rng(2)
    x = _bf16(rng.normal(size=(50, 384)))
    w = rng.uniform(0.01, 1.0, size=(50, 1)).astype(np.float32)
    ref = x * torch.from_numpy(w).to(torch.bfloat16)       # torch CPU bf16 arithmetic
    a, _ = oracle.prepare(_bits(x), w, True, "none")
    np.testing.assert_array_equal(a, _bits(ref))


def test_prepare_weight_on_input_requires_top1():
    with pytest.raises(ValueError):
        oracle.prepare(np.zeros((2, 128), np.uint16), np.ones((2, 2), np.float32), True)


def test_fp8_quantiser_matches_torch_float32_and_cast():
    rng = np.random.default_rng(3)
    x = _bf16(rng.normal(size=(40, 512)) * rng.uniform(0.01, 100, size=(40, 1)))
    q, s = oracle.prepare(_bits(x), None, False, "fp8")
    xf = x.float().view(40, 4, 128)
    amax = xf.abs().amax(dim=2)
    s_ref = torch.clamp(amax, min=1e-10) / 448.0                 # float32 torch ops
    q_ref = (xf / s_ref[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).view(40, 512)
    np.testing.assert_array_equal(s, s_ref.numpy())
    np.testing.assert_array_equal(q, q_ref.numpy())


def test_fp8_quantiser_closed_forms():
    row = np.zeros((3, 256), dtype=np.float64)
    row[0, :128] = 1.0          # constant group -> code 448, scale 1/448
    row[0, 128:] = -2.5
    row[1, :] = 0.0             # zero group -> code 0, scale 1e-10/448
    row[2, :128] = 448.0        # amax 448 -> scale exactly 1, codes = values
    row[2, 128:] = np.linspace(-3, 3, 128)
    q, s = oracle.quantize_g128(row)
    assert np.all(q[0, :128] == 0x7E) and np.all(q[0, 128:] == 0xFE)
    assert s[0, 0] == np.float32(1.0) / np.float32(448.0)
    assert s[0, 1] == np.float32(2.5) / np.float32(448.0)
    assert np.all(q[1] == 0) and s[1, 0] == np.float32(1e-10) / np.float32(448.0)
    assert s[2, 0] == 1.0 and np.all(q[2, :128] == 0x7E)


def test_fp8_round_trip_error_bound():
    rng = np.random.default_rng(4)
    v = rng.normal(size=(64, 1024)) * rng.uniform(1e-3, 1e3, size=(64, 1))
    q, s = oracle.quantize_g128(v)
    deq = oracle.dequant_g128(q, s)
    v32 = v.astype(np.float32).astype(np.float64)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    scaled = np.abs(v32) / srep
    normal = scaled >= 2.0 ** -6
    err = np.abs(deq - v32)
    # half an ulp of the 3-bit mantissa relative, plus the float32 rounding of v/s
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -22) * np.abs(v32[normal]))
    assert np.all(err[~normal] <= srep[~normal] * (2.0 ** -10 + 2.0 ** -30))
    amax_code = np.abs(codecs.e4m3_decode(q)).reshape(64, 8, 128).max(axis=2)
    assert np.all(amax_code == 448.0)       # every group's largest element hits the top code


def test_per_token_and_per_tensor_quantisers_match_torch_float32_and_cast():
    """The "A" and "T" formats: one scale per token row / for the whole
    tensor, same rule as G(128), checked against torch float32 ops + the
    float8_e4m3fn cast."""
    rng = np.random.default_rng(5)
    x = _bf16(rng.normal(size=(24, 384)) * rng.uniform(0.01, 100, size=(24, 1)))
    xf = x.float()
    q, s = oracle.prepare(_bits(x), None, False, "fp8_token")
    s_ref = torch.clamp(xf.abs().amax(dim=1, keepdim=True), min=1e-10) / 448.0
    assert s.shape == (24, 1)
    np.testing.assert_array_equal(s, s_ref.numpy())
    np.testing.assert_array_equal(q, (xf / s_ref).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    q, s = oracle.prepare(_bits(x), None, False, "fp8_tensor")
    s_ref = torch.clamp(xf.abs().amax(), min=1e-10).reshape(1, 1) / 448.0
    assert s.shape == (1, 1)
    np.testing.assert_array_equal(s, s_ref.numpy())
    np.testing.assert_array_equal(q, (xf / s_ref).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_scale_formats_nest():
    """A row's per-token scale is the largest of its G(128) scales, and the
    per-tensor scale the largest per-token scale (amax and the scale rule are
    monotone)."""
    rng = np.random.default_rng(6)
    v = rng.normal(size=(17, 640)) * rng.uniform(1e-3, 1e3, size=(17, 5)).repeat(128, axis=1)
    _, sg = oracle.quantize_g128(v)
    _, st = oracle.quantize_token(v)
    _, sT = oracle.quantize_tensor(v)
    np.testing.assert_array_equal(st[:, 0], sg.max(axis=1))
    assert sT[0, 0] == st.max()


def test_dequant_scaled_broadcasts_each_format():
    rng = np.random.default_rng(7)
    v = rng.normal(size=(6, 256))
    for quant in (oracle.quantize_g128, oracle.quantize_token, oracle.quantize_tensor):
        q, s = quant(v)
        deq = oracle.moe.dequant_scaled(q, s)
        full = np.broadcast_to(np.repeat(s, 128, axis=1) if s.shape[1] == 2 else s, v.shape)
        np.testing.assert_array_equal(deq, codecs.e4m3_decode(q) * full)
