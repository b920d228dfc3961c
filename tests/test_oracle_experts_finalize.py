"""Pins of the oracle's experts and finalize steps against torch CPU float64
(dense MLP, einsum over all experts then masked, F.rms_norm), closed forms,
exact scaling laws and the top-1 input-weighting identity."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import codecs


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f64(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16).double()


def _rand_bf16(rng, shape, std=1.0):
    return _bf16_bits(rng.normal(0, std, size=shape))


# ---------------------------------------------------------------- experts
def test_single_expert_top1_is_a_dense_swiglu_mlp():
    """E = 1, k = 1 reduces to one SwiGLU MLP: y = W2 (silu(W1 x) * (W3 x)).
    Non-square shapes catch a transposed operand; silu(g)*u != silu(u)*g
    catches swapped gate/up halves."""
    rng = np.random.default_rng(21)
    T, H, I = 9, 48, 20
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (1, 2 * I, H), 0.3)
    w2 = _rand_bf16(rng, (1, H, I), 0.3)
    ids = np.zeros((T, 1), np.int32)
    feo, _ = oracle.experts(x, None, ids, w13, None, w2, None, "silu", "exact")
    xt, W13, W2 = _f64(x), _f64(w13[0]), _f64(w2[0])
    ref = (F.silu(xt @ W13[:I].T) * (xt @ W13[I:].T)) @ W2.T
    np.testing.assert_array_equal(feo[:, 0], _bf16_bits(ref.numpy()))


def test_silu_no_mul_is_silu_then_down_projection():
    rng = np.random.default_rng(22)
    T, H, I = 7, 40, 24
    x = _rand_bf16(rng, (T, H))
    w1 = _rand_bf16(rng, (1, I, H), 0.3)
    w2 = _rand_bf16(rng, (1, H, I), 0.3)
    feo, _ = oracle.experts(x, None, np.zeros((T, 1), np.int32), w1, None, w2, None,
                            "silu_no_mul", "exact")
    ref = F.silu(_f64(x) @ _f64(w1[0]).T) @ _f64(w2[0]).T
    np.testing.assert_array_equal(feo[:, 0], _bf16_bits(ref.numpy()))


def test_gelu_closed_forms():
    """GELU(v) = v * Phi(v): the textbook value Phi(1) = 0.8413447460685429,
    GELU(v) - GELU(-v) = v (Phi(v) + Phi(-v) = 1), GELU(0) = 0, and
    GELU(v) -> v for large v."""
    g = oracle.moe.gelu
    assert g(0.0) == 0.0
    assert abs(g(1.0) - 0.8413447460685429) < 1e-15
    assert abs(g(-1.0) + 0.15865525393145707) < 1e-15
    v = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(g(v) - g(-v), v, rtol=0, atol=1e-14)
    assert abs(g(10.0) - 10.0) < 1e-20


def test_gelu_mul_single_expert_matches_torch_exact_gelu():
    """E = 1, k = 1 with the gated GELU: y = W2 (gelu(W1 x) * (W3 x)), with
    torch's erf-form GELU in float64 (not the tanh approximation)."""
    rng = np.random.default_rng(24)
    T, H, I = 9, 48, 20
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (1, 2 * I, H), 0.3)
    w2 = _rand_bf16(rng, (1, H, I), 0.3)
    feo, _ = oracle.experts(x, None, np.zeros((T, 1), np.int32), w13, None, w2, None, "gelu",
                            "exact")
    xt, W13, W2 = _f64(x), _f64(w13[0]), _f64(w2[0])
    ref = (F.gelu(xt @ W13[:I].T, approximate="none") * (xt @ W13[I:].T)) @ W2.T
    np.testing.assert_array_equal(feo[:, 0], _bf16_bits(ref.numpy()))
    # and not the tanh form, which differs by more than bf16 rounding here
    tanh = (F.gelu(xt @ W13[:I].T, approximate="tanh") * (xt @ W13[I:].T)) @ W2.T
    assert not np.array_equal(_bf16_bits(tanh.numpy()), feo[:, 0])


def test_gelu_no_mul_is_gelu_then_down_projection():
    rng = np.random.default_rng(25)
    T, H, I = 7, 40, 24
    x = _rand_bf16(rng, (T, H))
    w1 = _rand_bf16(rng, (1, I, H), 0.3)
    w2 = _rand_bf16(rng, (1, H, I), 0.3)
    feo, _ = oracle.experts(x, None, np.zeros((T, 1), np.int32), w1, None, w2, None,
                            "gelu_no_mul", "exact")
    ref = F.gelu(_f64(x) @ _f64(w1[0]).T) @ _f64(w2[0]).T
    np.testing.assert_array_equal(feo[:, 0], _bf16_bits(ref.numpy()))


def test_experts_match_dense_all_experts_then_mask():
    """Brute force: every expert on every token (one einsum over all experts),
    then pick each (token, slot) by topk_ids."""
    rng = np.random.default_rng(23)
    T, H, I, E, k = 13, 64, 32, 6, 3
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (E, 2 * I, H), 0.2)
    w2 = _rand_bf16(rng, (E, H, I), 0.2)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    feo, _ = oracle.experts(x, None, ids, w13, None, w2, None, "silu", "exact")
    xt, W13, W2 = _f64(x), _f64(w13), _f64(w2)
    h = torch.einsum("th,enh->ten", xt, W13)                      # [T, E, 2I]
    z = F.silu(h[..., :I]) * h[..., I:]
    y_all = torch.einsum("tei,edi->ted", z, W2)                   # [T, E, H]
    ref = torch.stack([y_all[t, torch.from_numpy(ids[t].astype(np.int64))] for t in range(T)])
    np.testing.assert_array_equal(feo, _bf16_bits(ref.numpy()))


def test_fp8_weight_dequant_uses_block_row_col_scales():
    """One 128x128 scale per block, indexed [n // 128, k // 128]: a
    non-square scale grid catches a transposed block index."""
    rng = np.random.default_rng(24)
    N, K = 256, 384
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    scales = np.arange(1, 7, dtype=np.float32).reshape(2, 3)
    deq = oracle.moe.dequant_weight(codes, scales)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for bn in range(2):
        for bk in range(3):
            blk = (slice(bn * 128, bn * 128 + 128), slice(bk * 128, bk * 128 + 128))
            np.testing.assert_array_equal(deq[blk], ref[blk] * scales[bn, bk])


def test_fp8_experts_match_torch_on_dequantised_operands():
    rng = np.random.default_rng(25)
    T, H, I, E, k = 11, 256, 128, 4, 2
    xq, xs = oracle.quantize_g128(rng.normal(size=(T, H)))
    w13 = rng.integers(0, 0x7E, size=(E, 2 * I, H), dtype=np.uint8)
    w2 = rng.integers(0, 0x7E, size=(E, H, I), dtype=np.uint8)
    s13 = rng.uniform(1e-3, 2e-3, size=(E, 2, 2)).astype(np.float32)
    s2 = rng.uniform(1e-3, 2e-3, size=(E, 2, 1)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    feo, _ = oracle.experts(xq, xs, ids, w13, s13, w2, s2, "silu", "exact")

    def deq(c, s):
        v = torch.from_numpy(c).view(torch.float8_e4m3fn).double()
        return v * torch.from_numpy(s).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    A = torch.from_numpy(xq).view(torch.float8_e4m3fn).double() * \
        torch.from_numpy(xs).double().repeat_interleave(128, 1)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            W13, W2 = deq(w13[e], s13[e]), deq(w2[e], s2[e])
            h = W13 @ A[t]
            y = W2 @ (F.silu(h[:I]) * h[I:])
            np.testing.assert_array_equal(feo[t, j], _bf16_bits(y.numpy()))


def test_down_projection_scaling_is_exact():
    """W2 * 2 doubles every expert output exactly (a power-of-two scaling
    commutes with every rounding)."""
    rng = np.random.default_rng(26)
    T, H, I, E, k = 10, 32, 16, 4, 2
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (E, 2 * I, H), 0.3)
    w2 = _rand_bf16(rng, (E, H, I), 0.3)
    w2x2 = _bf16_bits(codecs.bf16_bits_to_f64(w2) * 2.0)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    a, _ = oracle.experts(x, None, ids, w13, None, w2, None)
    b, _ = oracle.experts(x, None, ids, w13, None, w2x2, None)
    np.testing.assert_array_equal(codecs.bf16_bits_to_f64(b), 2.0 * codecs.bf16_bits_to_f64(a))


def test_shared_expert_equals_routed_expert_with_same_weights():
    rng = np.random.default_rng(27)
    T, H, I = 8, 64, 32
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (1, 2 * I, H), 0.3)
    w2 = _rand_bf16(rng, (1, H, I), 0.3)
    feo, sh = oracle.experts(x, None, np.zeros((T, 1), np.int32), w13, None, w2, None,
                             shared=dict(a=x, w13=w13[0], w2=w2[0]))
    np.testing.assert_array_equal(sh, feo[:, 0])


def test_token_subset_matches_full_run():
    rng = np.random.default_rng(28)
    T, H, I, E, k = 20, 32, 16, 5, 2
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (E, 2 * I, H), 0.3)
    w2 = _rand_bf16(rng, (E, H, I), 0.3)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    full, _ = oracle.experts(x, None, ids, w13, None, w2, None)
    sub = np.array([3, 7, 19])
    part, _ = oracle.experts(x, None, ids, w13, None, w2, None, tokens=sub)
    np.testing.assert_array_equal(part[sub], full[sub])


def test_mirrored_mode_differs_from_exact_by_rounding_only():
    rng = np.random.default_rng(29)
    T, H, I, E, k = 30, 128, 256, 4, 2
    x = _rand_bf16(rng, (T, H))
    w13 = _rand_bf16(rng, (E, 2 * I, H), 1 / np.sqrt(H))
    w2 = _rand_bf16(rng, (E, H, I), 1 / np.sqrt(I))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ex, _ = oracle.experts(x, None, ids, w13, None, w2, None, mode="exact")
    mi, _ = oracle.experts(x, None, ids, w13, None, w2, None, mode="mirrored")
    a, b = codecs.bf16_bits_to_f64(ex), codecs.bf16_bits_to_f64(mi)
    assert 0 < np.abs(a - b).max() <= 2e-2 * np.abs(a).max()


# ------------------------------------------------------- top-1 identity
def test_top1_weight_on_input_identity_for_a_linear_activation():
    """With a positively homogeneous activation (here the identity) and a
    power-of-two router weight, putting the weight on the input (finalize
    then uses weight 1) equals putting it on the output: bit-exact."""
    rng = np.random.default_rng(30)
    T, H, I, E = 12, 64, 32, 4
    x = _rand_bf16(rng, (T, H))
    w1 = _rand_bf16(rng, (E, I, H), 0.3)
    w2 = _rand_bf16(rng, (E, H, I), 0.3)
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    tw = (2.0 ** -rng.integers(0, 4, size=(T, 1))).astype(np.float32)
    lin = lambda h: h  # noqa: E731
    a_in, _ = oracle.prepare(x, tw, True)
    feo_in, _ = oracle.experts(a_in, None, ids, w1, None, w2, None, lin)
    out_in, _, _ = oracle.finalize(feo_in, tw, True)
    feo_out, _ = oracle.experts(x, None, ids, w1, None, w2, None, lin)
    out_out, _, _ = oracle.finalize(feo_out, tw, False)
    np.testing.assert_array_equal(out_in, out_out)
    # silu is not homogeneous: the same construction differs (reported, bounded)
    f_in, _ = oracle.experts(a_in, None, ids, w1, None, w2, None, "silu_no_mul")
    f_out, _ = oracle.experts(x, None, ids, w1, None, w2, None, "silu_no_mul")
    o_in = codecs.bf16_bits_to_f64(oracle.finalize(f_in, tw, True)[0])
    o_out = codecs.bf16_bits_to_f64(oracle.finalize(f_out, tw, False)[0])
    assert np.abs(o_in - o_out).max() > 0


def test_weight_on_input_with_unit_weight_is_identity():
    rng = np.random.default_rng(31)
    x = _rand_bf16(rng, (6, 128))
    a, _ = oracle.prepare(x, np.ones((6, 1), np.float32), True)
    np.testing.assert_array_equal(a, x)


# --------------------------------------------------------------- finalize
def test_finalize_matches_torch_rms_norm():
    rng = np.random.default_rng(32)
    T, k, H = 17, 4, 256
    y = _rand_bf16(rng, (T, k, H))
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    sh, res = _rand_bf16(rng, (T, H)), _rand_bf16(rng, (T, H))
    gamma = _bf16_bits(rng.uniform(0.5, 1.5, size=H))
    out, _, res_out = oracle.finalize(y, w, False, sh, res, gamma, 1e-6)
    acc = torch.einsum("tk,tkh->th", torch.from_numpy(w).double(), _f64(y)) + _f64(sh) + _f64(res)
    ref = F.rms_norm(acc, (H,), weight=_f64(gamma), eps=1e-6)
    np.testing.assert_array_equal(out, _bf16_bits(ref.numpy()))
    np.testing.assert_array_equal(res_out, _bf16_bits(acc.numpy()))


def test_finalize_plain_weighted_sum_without_fusions():
    rng = np.random.default_rng(33)
    y = _rand_bf16(rng, (9, 2, 64))
    w = rng.uniform(0, 1, size=(9, 2)).astype(np.float32)
    out, s, _ = oracle.finalize(y, w, False)
    ref = torch.einsum("tk,tkh->th", torch.from_numpy(w).double(), _f64(y))
    assert s is None
    np.testing.assert_array_equal(out, _bf16_bits(ref.numpy()))


def test_finalize_weight_on_input_ignores_weights():
    rng = np.random.default_rng(34)
    y = _rand_bf16(rng, (5, 1, 64))
    a, _, _ = oracle.finalize(y, np.full((5, 1), 0.3, np.float32), True)
    np.testing.assert_array_equal(a, y[:, 0])


def test_finalize_closed_forms():
    H = 128
    gamma = _bf16_bits(np.full(H, 1.5))
    # k = 1, w = 1, constant row c: out = c / sqrt(c^2 + eps) * gamma
    for c in (2.0, -0.75, 1e-3):
        y = _bf16_bits(np.full((1, 1, H), c))
        out, _, _ = oracle.finalize(y, np.ones((1, 1), np.float32), False, gamma=gamma, eps=1e-6)
        cb = codecs.bf16_bits_to_f64(y)[0, 0, 0]
        expect = cb / np.sqrt(cb * cb + 1e-6) * 1.5
        np.testing.assert_array_equal(codecs.bf16_bits_to_f64(out), np.full((1, H), codecs.bf16_bits_to_f64(_bf16_bits(expect))))
    # zero row stays zero
    z = np.zeros((1, 2, H), np.uint16)
    out, _, _ = oracle.finalize(z, np.full((1, 2), 0.5, np.float32), False, gamma=gamma)
    assert np.all(codecs.bf16_bits_to_f64(out) == 0)
    # identical rows with weights summing to one give the row back
    row = _rand_bf16(np.random.default_rng(35), (1, 1, H))
    y = np.repeat(row, 4, axis=1)
    out, _, _ = oracle.finalize(y, np.full((1, 4), 0.25, np.float32), False)
    np.testing.assert_array_equal(out[0], row[0, 0])


def test_finalize_fp8_output_matches_torch_quantisation():
    rng = np.random.default_rng(36)
    T, k, H = 6, 4, 512
    y = _rand_bf16(rng, (T, k, H))
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    gamma = _bf16_bits(rng.uniform(0.5, 1.5, size=H))
    q, s, _ = oracle.finalize(y, w, False, gamma=gamma, out_quant="fp8")
    acc = torch.einsum("tk,tkh->th", torch.from_numpy(w).double(), _f64(y))
    ref = F.rms_norm(acc, (H,), weight=_f64(gamma), eps=1e-6).float().view(T, H // 128, 128)
    s_ref = torch.clamp(ref.abs().amax(2), min=1e-10) / 448.0
    q_ref = (ref / s_ref[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).view(T, H)
    np.testing.assert_array_equal(s, s_ref.numpy())
    np.testing.assert_array_equal(q, q_ref.numpy())
