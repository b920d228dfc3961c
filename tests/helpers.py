"""Shared test utilities: tolerance checks and tensor <-> numpy plumbing."""

import numpy as np
import torch

from oracle import codecs
from workloads import to_numpy_bits

BF16_BOUND = 2e-2      # max|err| <= 2e-2 * max|ref| on the bf16 path
FP8_BOUND = 6e-2       # max|err| <= 6e-2 * max|ref| on the fp8 path
ELEM_REL = 5e-2        # per element, against the mirrored oracle, where |ref| > 1e-2
ELEM_FLOOR = 1e-2


def f64_of_bf16(x):
    """bf16 tensor or uint16 bits -> float64 numpy."""
    if isinstance(x, torch.Tensor):
        x = to_numpy_bits(x)
    return codecs.bf16_bits_to_f64(x)


def f64_of_fp8(codes, scales):
    """E4M3 codes [R, C] + G(128) scales [R, C/128] -> float64 numpy."""
    if isinstance(codes, torch.Tensor):
        codes = to_numpy_bits(codes)
    if isinstance(scales, torch.Tensor):
        scales = to_numpy_bits(scales)
    return codecs.e4m3_decode(codes) * np.repeat(np.asarray(scales, np.float64), 128, axis=-1)


def bf16_ulp(x):
    """Spacing of bf16 numbers just above |x| (x already bf16-representable):
    the size of a one-step rounding flip of that value."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    return np.where(x > 0, np.exp2(e - 7), np.exp2(-133.0))


def finalize_flip_allowance(ref, gamma_bits=None):
    """Per-output-element size of the rounding flips that the pages' bf16
    boundaries allow, from the mirrored oracle's forward() dict.

    Every routed row y[t, j] (and the shared row) is rounded to bf16 before
    the weighted reduction.  Two correct implementations accumulate the
    GEMM in different orders, so a value that lands within rounding error of
    a bf16 midpoint may round either way: y[t, j, h] may differ by one bf16
    step.  The reduction then moves by sum_j |w[t, j]| * ulp(y[t, j, h])
    (+ ulp of the shared row), scaled by the RMSNorm factor when gamma is
    given, and the final bf16 rounding adds one more step of the output.
    Where the reduction cancels, this is larger than 5 % of the result."""
    tok = ref["tokens"]
    y = f64_of_bf16(ref["fused_expert_output"])[tok]            # [n, k, H]
    w = np.abs(np.asarray(ref["topk_weights"], np.float64)[tok])  # [n, k]
    acc = (w[:, :, None] * bf16_ulp(y)).sum(axis=1)
    if ref.get("shared_out") is not None:
        acc += bf16_ulp(f64_of_bf16(ref["shared_out"])[tok])
    if gamma_bits is not None:
        racc = f64_of_bf16(ref["residual_out"])
        racc = racc[tok] if racc.shape[0] != tok.size else racc
        r = 1.0 / np.sqrt((racc * racc).mean(axis=1, keepdims=True) + 1e-12)
        acc = acc * r * np.abs(f64_of_bf16(gamma_bits))[None, :]
    return acc


def check_tolerance(got, ref_exact, ref_mirrored, path, what="", elementwise=True,
                    min_identical=None, allowance=None):
    """The parity bar for floating-point outputs: max-norm bound against both
    oracle modes, per-element relative bound against the mirrored mode.

    Per element (where |ref| > 1e-2): |got - ref| <= 5e-2 * |ref| + allowance,
    where ``allowance`` (default 0) is the size of the one-step bf16 rounding
    flips of intermediates that the pages fix in bf16 (finalize_flip_allowance).

    elementwise=False drops the per-element bound: used for end-to-end
    outputs downstream of the fp8 re-quantisation of the intermediate z,
    where two correct results legitimately differ by whole fp8 code steps at
    rounding edges; there the per-element bound is checked stage by stage
    (z codes within one step, GEMM-2 against the z it consumed).

    min_identical: if given, at least this fraction of elements must equal
    the mirrored oracle exactly (the bf16 path mirrors every rounding)."""
    bound = BF16_BOUND if path == "bf16" else FP8_BOUND
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    report = {}
    for name, ref in (("exact", ref_exact), ("mirrored", ref_mirrored)):
        if ref is None:
            continue
        ref = np.asarray(ref, np.float64)
        m = np.abs(ref).max() if ref.size else 0.0
        err = np.abs(got - ref).max() if ref.size else 0.0
        report[name] = err / m if m > 0 else err
        assert err <= bound * m + 1e-30, f"{what}: max|err| {err:.3g} > {bound} * max|ref| {m:.3g} ({name})"
    if elementwise and ref_mirrored is not None and np.asarray(ref_mirrored).size:
        ref = np.asarray(ref_mirrored, np.float64)
        allow = np.zeros_like(ref) if allowance is None else np.broadcast_to(allowance, ref.shape)
        mask = np.abs(ref) > ELEM_FLOOR
        if mask.any():
            err = np.abs(got - ref)[mask]
            lim = ELEM_REL * np.abs(ref)[mask] + allow[mask]
            worst = int(np.argmax(err / lim))
            report["elem_rel"] = float((err / np.abs(ref)[mask]).max())
            report["elem_frac_of_limit"] = float(err[worst] / lim[worst])
            assert np.all(err <= lim), (
                f"{what}: per-element err {err[worst]:.3g} > limit {lim[worst]:.3g} "
                f"(ref {ref[mask][worst]:.4g}, got {got[mask][worst]:.4g})")
    if min_identical is not None and ref_mirrored is not None and np.asarray(ref_mirrored).size:
        same = float((got == np.asarray(ref_mirrored, np.float64)).mean())
        report["identical"] = same
        assert same >= min_identical, f"{what}: only {same:.3f} of elements equal the mirrored oracle"
    return report


def np_bits(t):
    return to_numpy_bits(t)


def e4m3_step(v):
    """Distance from |v| (an E4M3 value) to its next code up: 2^-9 below 2^-6,
    else 2^(floor(log2 |v|) - 3)."""
    a = np.abs(np.asarray(v, np.float64))
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))
    return np.ldexp(1.0, ex - 1 - 3)


# The kernel's z is an fp32 sum over H with per-128 block-scale promotions,
# accumulated inside the fp8 matrix unit in its own order; measured on the
# MI355X its absolute error reaches ~3.5e-5 of the group's amax (an fp32
# emulation of the same blocking stays below 3e-7).  Codes near zero may
# therefore differ by up to 1e-4 * amax = 0.0448 code units (448 units =
# amax), i.e. ~23 E4M3 subnormal steps; larger codes by one step.
Z_CODE_FLOOR = 1e-4 * 448.0


def check_fp8_codes(q_got, s_got, z_ref, what=""):
    """GPU E4M3 G(128) codes/scales of an fp32 quantity against the oracle's
    quantisation of its own float64 value: scales agree to 1e-4, and each
    code is the oracle's, its neighbour (the values straddled a rounding
    edge), or -- near zero -- within the fp32 accumulation floor.  Returns
    the fraction of identical codes."""
    import oracle
    q_ref, s_ref = oracle.quantize_g128(z_ref)
    np.testing.assert_allclose(s_got, s_ref, rtol=1e-4, err_msg=f"{what}: z scales")
    vg = codecs.e4m3_decode(q_got)
    vr = codecs.e4m3_decode(q_ref)
    tol = np.maximum(e4m3_step(np.maximum(np.abs(vg), np.abs(vr))), Z_CODE_FLOOR) + 1e-12
    bad = np.abs(vg - vr) > tol
    assert not bad.any(), f"{what}: {bad.sum()} z codes beyond one step / the accumulation floor"
    return float((q_got == q_ref).mean())
