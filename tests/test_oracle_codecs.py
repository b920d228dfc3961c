"""Pins of the oracle's number formats against torch's CPU casts (a library
routine independent of the oracle) and the formats' closed forms."""

import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_random_bit_patterns():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = codecs.f64_to_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(ours, _torch_bf16_bits(x))


def test_bf16_rne_ties_and_subnormals():
    rng = np.random.default_rng(12)
    hi = rng.integers(0, 2 ** 16, size=50_000, dtype=np.uint32)
    # exact ties (low half 0x8000), one above, one below; plus subnormals
    for low in (0x8000, 0x8001, 0x7FFF, 0x0000):
        x = ((hi << 16) | low).astype(np.uint32).view(np.float32)
        x = x[np.isfinite(x)]
        np.testing.assert_array_equal(codecs.f64_to_bf16_bits(x.astype(np.float64)),
                                      _torch_bf16_bits(x))
    sub = (rng.integers(1, 2 ** 23, size=10_000, dtype=np.uint32)).view(np.float32)
    np.testing.assert_array_equal(codecs.f64_to_bf16_bits(sub.astype(np.float64)),
                                  _torch_bf16_bits(sub))


def test_bf16_decode_matches_torch_for_all_finite_patterns():
    bits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = codecs.bf16_bits_to_f64(bits)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_bf16_overflow_goes_to_inf():
    big = np.array([3.5e38, -3.5e38, np.ldexp(2.0 - 2.0 ** -8, 127)], dtype=np.float64)
    out = codecs.f64_to_bf16_bits(big)
    assert list(out) == [0x7F80, 0xFF80, 0x7F80]


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])


def test_e4m3_closed_form_landmarks():
    d = codecs.e4m3_decode(np.array([0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE, 0x80], dtype=np.uint8))
    assert list(d[:6]) == [2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 448.0, -448.0]
    assert d[6] == 0.0 and np.signbit(d[6])


def _positive_grid():
    v = codecs.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    return np.sort(v)


def test_e4m3_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(13)
    x = np.concatenate([
        rng.normal(0, 50, 100_000), rng.normal(0, 0.01, 50_000),
        rng.uniform(-463.9, 463.9, 50_000), rng.normal(0, 2.0 ** -8, 20_000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codecs.e4m3_encode_sat(x.astype(np.float64)), ref)


def test_e4m3_encode_ties_to_even_matches_torch():
    g = _positive_grid()
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)   # exact midpoints, representable in f32
    x = np.concatenate([mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = codecs.e4m3_encode_sat(x.astype(np.float64))
    np.testing.assert_array_equal(ours, ref)
    # ties go to the even code
    assert np.all(ours[: mids.size] % 2 == 0)


def test_e4m3_encode_saturates():
    x = np.array([464.0, 480.0, 1e6, -500.0, -1e30, 447.9], dtype=np.float64)
    assert list(codecs.e4m3_encode_sat(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E]


@pytest.mark.parametrize("code", list(range(0, 0x7F)))
def test_e4m3_round_trip_every_code(code):
    v = codecs.e4m3_decode(np.array([code, code | 0x80], dtype=np.uint8))
    back = codecs.e4m3_encode_sat(v)
    assert list(back) == [code, code | 0x80]
