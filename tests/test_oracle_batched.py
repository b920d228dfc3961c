"""Pins of the oracle's batched-format experts stage (oracle.experts_batched).

The batched stage runs the same per-row MLP as the standard stage, so it is
pinned by
  * a closed form: identity weights turn the MLP into an elementwise
    function of the input row, evaluated here with torch's float64 SiLU/GELU,
    with a different gate gain per expert (a row read from or written to the
    wrong batch fails);
  * the standard-format stage (pinned on its own in test_oracle_experts_*):
    scattering the routed rows of a top-k routing into per-expert batches, in
    flat-row order, must give back the standard output row for row;
  * the format rules: rows past a count stay zero, counts are clamped to
    [0, M], a per-tensor scale [1, 1] equals the same value per row, a subset
    of experts reproduces those experts' batches of the full run.
"""

import numpy as np
import torch

import oracle
from oracle import moe as om


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def test_closed_form_identity_weights():
    rng = np.random.default_rng(7)
    E, M, H = 3, 5, 128
    I = H
    gains = [0.5, 2.0, -1.0]
    a = _bf16(rng.standard_normal((E, M, H)))
    eye = np.eye(H)
    w13 = np.stack([np.concatenate([g * eye, eye]) for g in gains])       # gate = g a, up = a
    w2 = np.stack([eye] * E)
    counts = np.array([5, 2, 0], np.int32)
    for act, fn in (("silu", torch.nn.functional.silu),
                    ("gelu", lambda v: torch.nn.functional.gelu(v, approximate="none"))):
        out = oracle.experts_batched(a, None, counts, _bf16(w13), None, _bf16(w2), None, act)
        for e in range(E):
            v = torch.from_numpy(_f64(a[e]))
            want = _bf16((fn(gains[e] * v) * v).numpy())
            c = counts[e]
            np.testing.assert_array_equal(out[e, :c], want[:c])
            assert not out[e, c:].any()
    # ungated: W1 = g * Id only
    w1 = np.stack([g * eye for g in gains])
    out = oracle.experts_batched(a, None, counts, _bf16(w1), None, _bf16(w2), None, "silu_no_mul")
    for e in range(E):
        want = _bf16(torch.nn.functional.silu(gains[e] * torch.from_numpy(_f64(a[e]))).numpy())
        np.testing.assert_array_equal(out[e, :counts[e]], want[:counts[e]])


def _scatter(ids, E):
    """(expert, position) of every flat row i = t*k + j, rows of an expert in
    ascending i -- the order a dispatch that walks the tokens would fill."""
    flat = ids.reshape(-1)
    pos = np.zeros_like(flat)
    seen = np.zeros(E, np.int64)
    for i, e in enumerate(flat):
        pos[i] = seen[e]
        seen[e] += 1
    return flat, pos, seen


def _layer(rng, T, H, I, E, quant):
    x = _bf16(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w13 = _bf16(rng.standard_normal((E, 2 * I, H)) / np.sqrt(H))
    w2 = _bf16(rng.standard_normal((E, H, I)) / np.sqrt(I))
    return x, logits, w13, w2


def test_scatter_of_standard_rows_matches_standard_stage():
    rng = np.random.default_rng(11)
    T, H, I, E, k = 23, 256, 128, 6, 2
    x, logits, w13, w2 = _layer(rng, T, H, I, E, "none")
    ids, w = oracle.route(logits, k)
    for quant in ("none", "fp8", "fp8_token"):
        a1q, a1s = oracle.prepare(x, w, False, quant)
        if quant == "none":
            W13, S13, W2, S2 = w13, None, w2, None
        else:
            # fp8 weights: E4M3 codes of the bf16 draws with unit block scales
            W13 = oracle.e4m3_encode_sat(_f64(w13) * 64)
            W2 = oracle.e4m3_encode_sat(_f64(w2) * 64)
            S13 = np.full((E, 2 * I // 128, H // 128), 1 / 64, np.float32)
            S2 = np.full((E, H // 128, I // 128), 1 / 64, np.float32)
        for mode in ("exact", "mirrored"):
            std, _ = oracle.experts(a1q, a1s, ids, W13, S13, W2, S2, "silu", mode)
            flat, pos, counts = _scatter(ids, E)
            M = int(counts.max()) + 3
            a = np.zeros((E, M, H), a1q.dtype)
            a[flat, pos] = a1q[np.arange(T * k) // k]
            s = None
            if a1s is not None:
                s = np.zeros((E, M, a1s.shape[1]), np.float32)
                s[flat, pos] = a1s[np.arange(T * k) // k]
            out = oracle.experts_batched(a, s, counts, W13, S13, W2, S2, "silu", mode)
            np.testing.assert_array_equal(out[flat, pos], std.reshape(T * k, H))
            live = np.zeros((E, M), bool)
            live[flat, pos] = True
            assert not out[~live].any()


def test_counts_clamped_and_subset():
    rng = np.random.default_rng(3)
    E, M, H, I = 4, 6, 128, 128
    a = _bf16(rng.standard_normal((E, M, H)))
    w13 = _bf16(rng.standard_normal((E, 2 * I, H)) / np.sqrt(H))
    w2 = _bf16(rng.standard_normal((E, H, I)) / np.sqrt(I))
    full = oracle.experts_batched(a, None, [-3, M + 5, 2, M], w13, None, w2, None)
    same = oracle.experts_batched(a, None, [0, M, 2, M], w13, None, w2, None)
    np.testing.assert_array_equal(full, same)
    assert not full[0].any() and full[1].any() and not full[2, 2:].any()
    sub = oracle.experts_batched(a, None, [0, M, 2, M], w13, None, w2, None, experts_subset=[2])
    np.testing.assert_array_equal(sub[2], same[2])
    assert not sub[[0, 1, 3]].any()


def test_per_tensor_scale_broadcasts_like_rows():
    rng = np.random.default_rng(5)
    E, M, H, I = 3, 4, 256, 128
    codes = oracle.e4m3_encode_sat(rng.standard_normal((E, M, H)) * 100)
    w13 = oracle.e4m3_encode_sat(rng.standard_normal((E, 2 * I, H)) * 100)
    w2 = oracle.e4m3_encode_sat(rng.standard_normal((E, H, I)) * 100)
    s13 = np.full((E, 2 * I // 128, H // 128), 1e-3, np.float32)
    s2 = np.full((E, H // 128, I // 128), 2e-3, np.float32)
    counts = [4, 1, 3]
    t = oracle.experts_batched(codes, np.array([[0.01]], np.float32), counts, w13, s13, w2, s2)
    r = oracle.experts_batched(codes, np.full((E, M, 1), 0.01, np.float32), counts, w13, s13, w2,
                               s2)
    g = oracle.experts_batched(codes, np.full((E, M, H // 128), 0.01, np.float32), counts, w13,
                               s13, w2, s2)
    np.testing.assert_array_equal(t, r)
    np.testing.assert_array_equal(t, g)
    # a scale is a plain factor on the input: doubling it doubles the
    # gate and the up projections, so silu-mul output changes (not linear)
    d = oracle.experts_batched(codes, np.array([[0.02]], np.float32), counts, w13, s13, w2, s2)
    assert not np.array_equal(d, t)
    assert om.dequant_act(codes[0, :1], np.array([[0.02]]))[0, 0] == \
        2 * om.dequant_act(codes[0, :1], np.array([[0.01]]))[0, 0]
