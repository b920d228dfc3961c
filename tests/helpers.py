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


def check_tolerance(got, ref_exact, ref_mirrored, path, what=""):
    """The parity bar for floating-point outputs: max-norm bound against both
    oracle modes, per-element relative bound against the mirrored mode."""
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
    if ref_mirrored is not None and np.asarray(ref_mirrored).size:
        ref = np.asarray(ref_mirrored, np.float64)
        mask = np.abs(ref) > ELEM_FLOOR
        if mask.any():
            rel = np.abs(got - ref)[mask] / np.abs(ref)[mask]
            report["elem_rel"] = rel.max()
            assert rel.max() <= ELEM_REL, f"{what}: per-element rel err {rel.max():.3g} > {ELEM_REL}"
    return report


def np_bits(t):
    return to_numpy_bits(t)
