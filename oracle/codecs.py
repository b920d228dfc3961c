"""Number-format codecs for the CPU oracle (test infrastructure only).

bf16 is the storage type of activations and expert outputs; the pages fix
that the modular experts and finalize work in "the original activation
dtype" (Fused MoE Kernel Features, fused-experts section) and that kernels
run in float16/bfloat16 when no quant type is given (same page, backend
section).  fp8 is OCP E4M3 ("e4m3fn": bias 7, no infinities, 0x7F/0xFF NaN,
largest finite 448), the format of the G(128) per-token-group activation
quantisation the pages list for fp8 ("G(128)" in both tables' key).

All rounding is round-to-nearest, ties-to-even, computed in float64 where
every intermediate is exact: a value x is divided by the power-of-two quantum
of its binade (exact), rounded with numpy's ties-to-even ``rint`` and scaled
back (exact).
"""

import numpy as np

BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))
E4M3_MAX = 448.0


def _round_to_binary(x, p, emin):
    """Round float64 ``x`` to nearest-even in a binary format with ``p``
    significand bits (implicit bit included) and smallest normal exponent
    ``emin``; the exponent range is unbounded above (overflow is the
    caller's business).  Exact: only power-of-two scalings and ``rint``."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)            # ax = m * 2**ex with m in [0.5, 1)
    lead = np.where(ax == 0.0, emin, np.maximum(ex - 1, emin))
    quantum = np.ldexp(np.ones_like(x), lead - (p - 1))
    return np.rint(x / quantum) * quantum


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> bf16 bit patterns with one round-to-nearest-even.
    Overflow goes to +-inf, NaN to the quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_binary(x, 8, -126)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
    r32 = r.astype(np.float32)      # exact: r is a bf16 value (or inf)
    out = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), out).astype(np.uint16)


def _e4m3_closed_form(codes):
    """OCP E4M3 codes -> float64 by the format's closed form: sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 is
    subnormal (mantissa * 2**-9); 0x7F/0xFF are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9,
                   (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64)))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


# The closed form evaluated once on all 256 codes; decoding is a lookup.
_E4M3_VALUES = _e4m3_closed_form(np.arange(256, dtype=np.uint8))


def e4m3_decode(codes):
    """OCP E4M3 codes (uint8) -> float64: the closed form above, looked up."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_sat(x):
    """float64 -> OCP E4M3 codes: round-to-nearest-even, saturating to
    +-448 (the largest finite value).  The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_binary(x, 4, -6)
    r = np.clip(r, -E4M3_MAX, E4M3_MAX)
    a = np.abs(r)
    sign = np.where(np.signbit(x), 0x80, 0x00)
    _, ex = np.frexp(a)
    lead = ex - 1
    sub = a < 2.0 ** -6
    # Subnormal: mantissa counts multiples of 2**-9.
    code_sub = np.rint(a / 2.0 ** -9).astype(np.int64)
    # Normal: exponent field lead+7, mantissa (a/2**lead - 1) * 8.
    lead_n = np.where(sub, 0, lead)
    man = np.rint((a / np.ldexp(np.ones_like(a), lead_n) - 1.0) * 8.0)
    code_norm = ((lead_n + 7) << 3) | man.astype(np.int64)
    code = np.where(sub, code_sub, code_norm)
    return (code | sign).astype(np.uint8)
