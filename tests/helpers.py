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


def finalize_flip_allowance(ref, gamma_bits=None, weight_on_input=False):
    """Per-output-element size of the rounding flips that the pages' bf16
    boundaries allow, from the mirrored oracle's forward() dict.

    Every routed row y[t, j] (and the shared row) is rounded to bf16 before
    the weighted reduction.  Two correct implementations accumulate the
    GEMM in different orders, so a value that lands within rounding error of
    a bf16 midpoint may round either way: y[t, j, h] may differ by one bf16
    step.  The reduction then moves by sum_j |w[t, j]| * ulp(y[t, j, h])
    (+ ulp of the shared row), scaled by the RMSNorm factor when gamma is
    given, and the final bf16 rounding adds one more step of the output.
    Where the reduction cancels, this is larger than 5 % of the result.
    With the router weight on the input, finalize weights the row by 1
    (weight_on_input=True), not by the router weight."""
    tok = ref["tokens"]
    y = f64_of_bf16(ref["fused_expert_output"])[tok]            # [n, k, H]
    w = np.abs(np.asarray(ref["topk_weights"], np.float64)[tok])  # [n, k]
    if weight_on_input:
        w = np.ones_like(w)
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
                    min_identical=None, allowance=None, maxnorm_slack=None):
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
    the mirrored oracle exactly (the bf16 path mirrors every rounding).

    maxnorm_slack: per element, what a final rounding of the output may add
    on top of the max-norm bound (the bound applies to the value before its
    fp8 output rounding; output_allowance derives the slack)."""
    bound = BF16_BOUND if path == "bf16" else FP8_BOUND
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    report = {}
    for name, ref in (("exact", ref_exact), ("mirrored", ref_mirrored)):
        if ref is None:
            continue
        ref = np.asarray(ref, np.float64)
        m = np.abs(ref).max() if ref.size else 0.0
        diff = np.abs(got - ref)
        if maxnorm_slack is not None and ref.size:
            diff = np.maximum(diff - np.broadcast_to(maxnorm_slack, diff.shape), 0.0)
        err = diff.max() if ref.size else 0.0
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


def act_scale_k(a_scale, rows, K):
    """An fp8 activation's scales as one scale per (row, 128-deep k-tile)
    [rows, K/128], from G(128) [rows, K/128], per token [rows] / [rows, 1]
    or per tensor [1] / [1, 1] scales."""
    s = np.asarray(a_scale, np.float64)
    s = s.reshape(s.shape[0], -1)
    return np.broadcast_to(s, (rows, K // 128)) if s.shape[1] == 1 else s


def weight_scale_k(w_scale, N):
    """128x128 block scales [N/128, K/128] -> one scale per (row n, k-tile)."""
    return np.repeat(np.asarray(w_scale, np.float64), 128, axis=0)[:N]


def fp8_first_gemm_reference(qa, sa_k, w13_codes, w13_scale, activation):
    """Exact z of the fp8 first GEMM and a bound on the GPU's float32 z.

    h = (qa sa) (qw sw)^T in float64; |h_gpu - h| is what the fp8
    instruction's cut does to these operands plus the float32 sums
    (fp8_gemm_model_error), or, when there are too many products to model,
    the worst-case bound (fp8_gemm_error_bound); it carries through the
    activation (z_error_bound).  Returns (z, dz)."""
    from exact_inputs import fp8_gemm_error_bound, fp8_gemm_model_error, z_error_bound
    import oracle.moe as om
    qw = codecs.e4m3_decode(w13_codes)
    sw_k = weight_scale_k(w13_scale, qw.shape[0])
    h = (qa * np.repeat(sa_k, 128, axis=1)) @ (qw * np.repeat(sw_k, 128, axis=1)).T
    dh = fp8_gemm_model_error(qa, sa_k, qw, sw_k)
    if dh is None:                       # too many products to model: the bound
        dh = fp8_gemm_error_bound(qa, sa_k, qw, sw_k)
    fn = om.silu if activation.startswith("silu") else om.gelu
    if activation in ("silu", "gelu"):
        inter = qw.shape[0] // 2
        g, u = h[:, :inter], h[:, inter:]
        return fn(g) * u, z_error_bound(g, u, dh[:, :inter], dh[:, inter:])
    return fn(h), z_error_bound(h, None, dh, None)


def check_fp8_z(q_got, s_got, z_exact, dz, what=""):
    """GPU E4M3 G(128) codes and scales of z against the exact z, per element:
    the GPU holds z_gpu with |z_gpu - z| <= dz (fp8_first_gemm_reference) and
    stores RNE(z_gpu / s_gpu), so its dequantised value lies within dz plus
    half a code step of z; the scale s_gpu = amax_gpu / 448 lies within the
    group's largest dz / 448 of the exact one.  Returns the fraction of codes
    equal to the oracle's quantisation of the exact z."""
    import oracle
    q_got = np.asarray(q_got)
    s_rep = np.repeat(np.asarray(s_got, np.float64), 128, axis=1)
    v = codecs.e4m3_decode(q_got)
    deq = v * s_rep
    half = 0.5 * e4m3_step(v) * s_rep
    err = np.abs(deq - z_exact)
    lim = dz + half + 1e-6 * np.abs(z_exact) + 1e-30
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} z values beyond the derived bound; worst {(err / lim)[i]:.6g} of "
            f"its limit at {i}: z {z_exact[i]:.9g} dz {dz[i]:.4g} gpu {deq[i]:.9g} "
            f"(code {v[i]:g} x scale {s_rep[i]:.9g}) half step {half[i]:.4g}")
    R, C = z_exact.shape
    amax = np.abs(z_exact).reshape(R, C // 128, 128).max(-1)
    dmax = dz.reshape(R, C // 128, 128).max(-1)
    s_err = np.abs(np.asarray(s_got, np.float64) * 448.0 - amax)
    assert np.all(s_err <= dmax + 1e-6 * amax + 1e-30), f"{what}: z scales beyond the bound"
    q_ref, _ = oracle.quantize_g128(z_exact)
    return float((q_got == q_ref).mean())


def check_fp8_second_gemm(y_got_bits, qz, s_z, w2_codes, w2_scale, what=""):
    """GEMM-2 given the z the GPU consumed, per element: y = (qz sz)(qw sw)^T
    exactly; the GPU's float32 y lies within what the fp8 instruction's cut
    and the float32 sums do to it (fp8_gemm_model_error, or the worst-case
    bound at sizes too large to model) and is rounded to bf16 once.  Returns
    the fraction equal to bf16(y)."""
    from exact_inputs import fp8_gemm_error_bound, fp8_gemm_model_error
    qzv = codecs.e4m3_decode(qz)
    sz_k = act_scale_k(s_z, qzv.shape[0], qzv.shape[1])
    qw = codecs.e4m3_decode(w2_codes)
    sw_k = weight_scale_k(w2_scale, qw.shape[0])
    y = (qzv * np.repeat(sz_k, 128, axis=1)) @ (qw * np.repeat(sw_k, 128, axis=1)).T
    dy = fp8_gemm_model_error(qzv, sz_k, qw, sw_k)
    if dy is None:
        dy = fp8_gemm_error_bound(qzv, sz_k, qw, sw_k)
    got = codecs.bf16_bits_to_f64(y_got_bits)
    lim = dy + 0.5 * bf16_ulp(np.abs(y) + dy) + 1e-30
    err = np.abs(got - y)
    assert np.all(err <= lim), (f"{what}: {(err > lim).sum()} outputs beyond the derived bound; "
                                f"worst {(err / lim).max():.3g} of its limit")
    return float((got == codecs.bf16_bits_to_f64(codecs.f64_to_bf16_bits(y))).mean())


def bf16_gemm_error_bound(a, w, chunk=16):
    """Bound on |GPU float32 result - exact| for C = a w^T on the bf16 path.

    The bf16 matrix instruction adds its chunk of products (16 of K; 32 for
    the 16x16 shape, which only halves the count) to the accumulator with
    float32 rounding, in ascending K (the instruction shows no cut: its
    results stay within a rounding or two of the exact sum), so with
    prefix sums S_i at the chunk boundaries and u = 2^-24 the error is at
    most 2u (sum_i |S_i| + sum_k |a_k w_k|); a K split restarts the prefix
    sums and adds them up at the end, at most doubling that: 4u (...)."""
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    M, K = a.shape
    N = w.shape[0]
    out = np.empty((M, N))
    for n0 in range(0, N, 1024):
        wb = w[n0:n0 + 1024]
        acc = np.zeros((M, wb.shape[0]))
        tot = np.zeros_like(acc)
        for k0 in range(0, K, chunk):
            acc += a[:, k0:k0 + chunk] @ wb[:, k0:k0 + chunk].T
            tot += np.abs(acc)
        out[:, n0:n0 + 1024] = 4.0 * 2.0 ** -24 * (tot + np.abs(a) @ np.abs(wb).T)
    return out


def _first_gemm_reference(spec, a_rows, a_scale_rows, w13, w13_scale):
    """(exact z, bound on |z_gpu - z|) of the first GEMM for some rows, on
    either path."""
    from exact_inputs import z_error_bound
    import oracle.moe as om
    if spec.quant.startswith("fp8"):
        return fp8_first_gemm_reference(codecs.e4m3_decode(a_rows),
                                        act_scale_k(a_scale_rows, a_rows.shape[0], spec.H),
                                        w13, w13_scale, spec.activation)
    A = codecs.bf16_bits_to_f64(a_rows)
    W = codecs.bf16_bits_to_f64(w13)
    h = A @ W.T
    dh = bf16_gemm_error_bound(A, W)
    fn = om.silu if spec.activation.startswith("silu") else om.gelu
    if spec.activation in ("silu", "gelu"):
        inter = W.shape[0] // 2
        g, u = h[:, :inter], h[:, inter:]
        return fn(g) * u, z_error_bound(g, u, dh[:, :inter], dh[:, inter:])
    return fn(h), z_error_bound(h, None, dh, None)


def routed_allowance(spec, ref, hw, gamma_bits=None):
    """Per-element allowance of the GPU's bf16 output against the mirrored
    oracle's (``ref``: oracle.forward's dict, mode "mirrored"), derived from
    the rounding boundaries the path fixes and bounds on the GPU's float32
    sums (bf16_gemm_error_bound; fp8: the instruction's cut,
    fp8_gemm_error_bound):

      * z: the GPU holds z_gpu within dz of the exact z and stores it
        rounded (bf16, or E4M3 with s_gpu within max_group(dz)/448 of the
        exact scale); its stored value differs from the oracle's by at most
        the gap between the roundings of z - dz and z + dz and the oracle's
        (0 wherever that interval holds no rounding midpoint);
      * y = GEMM-2: that z gap times |W2|, plus the second GEMM's own bound
        and one bf16 step of y (rounded once on each side);
      * finalize: sum_j |w'_j| (w' = 1 with the weight on the input) times
        the y allowance of slot j (+ the shared row's), times the RMSNorm
        factor when gamma is given, plus one bf16 step of the output.
    ``ref`` must also carry "x_bits" (the layer input) when the router weight
    went on the input and there is a shared expert.  Returns an array shaped
    like the output rows of ref["tokens"]."""
    from exact_inputs import fp8_gemm_error_bound, fp8_gemm_model_error
    import oracle
    import oracle.moe as om
    fp8 = spec.quant.startswith("fp8")
    tok = np.asarray(ref["tokens"])
    k, H = spec.top_k, spec.H
    ids = np.asarray(ref["topk_ids"])[tok]

    def rows_allowance(a_rows, a_scale_rows, w13, s13, w2, s2):
        z, dz = _first_gemm_reference(spec, a_rows, a_scale_rows, w13, s13)
        R, C = z.shape
        W2 = np.abs(om.dequant_weight(w2, s2))
        if fp8:
            q_ref, s_ref = oracle.quantize_g128(z)
            s = np.repeat(s_ref.astype(np.float64), 128, axis=1)
            ds = np.repeat(dz.reshape(R, C // 128, 128).max(-1) / 448.0, 128, axis=1)
            az = np.abs(z)
            lo = np.maximum(az - dz, 0.0) / (s + ds)
            hi = (az + dz) / np.maximum(s - ds, 1e-300)
            v_ref = np.abs(codecs.e4m3_decode(q_ref)) * s
            v_lo = codecs.e4m3_decode(codecs.e4m3_encode_sat(np.minimum(lo, 448.0))) * (s - ds)
            v_hi = codecs.e4m3_decode(codecs.e4m3_encode_sat(np.minimum(hi, 448.0))) * (s + ds)
            dzq = np.maximum(np.abs(v_hi - v_ref), np.abs(v_ref - v_lo))
            qz = codecs.e4m3_decode(q_ref)
            zq = qz * s
            args = (qz, act_scale_k(s_ref, R, C), codecs.e4m3_decode(w2), weight_scale_k(s2, H))
            dy = fp8_gemm_model_error(*args)
            dy = fp8_gemm_error_bound(*args) if dy is None else dy
        else:
            rb = lambda v: codecs.bf16_bits_to_f64(codecs.f64_to_bf16_bits(v))   # noqa: E731
            zq = rb(z)
            dzq = np.maximum(np.abs(rb(z + dz) - zq), np.abs(zq - rb(z - dz)))
            dy = bf16_gemm_error_bound(zq, om.dequant_weight(w2, None))
        spread = dzq @ W2.T
        y = np.abs(zq @ om.dequant_weight(w2, s2).T)
        return spread + dy + bf16_ulp(y + dy + spread)

    a_all, s_all = ref["a1q"], ref["a1q_scale"]
    allow = np.zeros((tok.size, k, H))
    for e in np.unique(ids):
        rr, jj = np.nonzero(ids == e)
        t = tok[rr]
        allow[rr, jj] = rows_allowance(a_all[t], None if s_all is None else _rows(s_all, t),
                                       hw["w13"][e], hw["w13_scale"][e] if fp8 else None,
                                       hw["w2"][e], hw["w2_scale"][e] if fp8 else None)
    w = (np.ones((tok.size, k)) if spec.apply_router_weight_on_input
         else np.abs(np.asarray(ref["topk_weights"], np.float64)[tok]))
    acc = (w[:, :, None] * allow).sum(axis=1)
    if "shared_w13" in hw:
        # the shared expert reads the unweighted input (a1q unless the weight
        # went on the input)
        if spec.apply_router_weight_on_input:
            sa, ss = oracle.prepare(ref["x_bits"], None, False, spec.quant)
        else:
            sa, ss = a_all, s_all
        acc += rows_allowance(sa[tok], None if ss is None else _rows(ss, tok), hw["shared_w13"],
                              hw.get("shared_w13_scale"), hw["shared_w2"], hw.get("shared_w2_scale"))
    if gamma_bits is not None:
        racc = f64_of_bf16(ref["residual_out"])
        racc = racc[tok] if racc.shape[0] != tok.size else racc
        r = 1.0 / np.sqrt((racc * racc).mean(axis=1, keepdims=True) + 1e-12)
        acc = acc * r * np.abs(f64_of_bf16(gamma_bits))[None, :]
    out = f64_of_bf16(ref["output"])
    out = out[tok] if out.shape[0] != tok.size else out
    return acc + bf16_ulp(np.abs(out) + acc)


def _rows(scale, t):
    """Rows t of an activation-scale array (a per-tensor [1, 1] serves all)."""
    scale = np.asarray(scale)
    return scale if scale.shape[0] == 1 else scale[t]


def output_allowance(spec, ref, d, hw):
    """(per-element allowance, per-element max-norm slack) of the layer's
    output against the mirrored oracle (``ref``: oracle.forward's dict),
    from routed_allowance.  A bf16 output needs no max-norm slack.  An fp8
    output is RNE(out / s) with s = amax / 448 per 128-group: where the
    bounded interval of the GPU's pre-rounding value (the oracle's, +- the
    routed allowance) holds a rounding midpoint, the code may be the
    neighbour, one E4M3 step (up to 32/448 of the group amax, more than the
    6 % max-norm bound); the slack is that step there and 0 elsewhere."""
    import oracle
    gamma = to_numpy_bits(d.get("gamma"))
    ref = dict(ref, x_bits=to_numpy_bits(d["x"]))
    allow = routed_allowance(spec, ref, hw, gamma)
    if spec.out_quant != "fp8":
        return allow, None
    tok = np.asarray(ref["tokens"])
    pre, _, _ = oracle.finalize(ref["fused_expert_output"], ref["topk_weights"],
                                spec.apply_router_weight_on_input, ref["shared_out"],
                                to_numpy_bits(d.get("residual")), gamma, spec.eps, "none",
                                tokens=tok)
    v = np.abs(f64_of_bf16(pre))
    dv = allow + bf16_ulp(v)                  # the bf16 proxy of the pre-rounding value
    R, C = v.shape
    s_ref = np.repeat(np.asarray(ref["output_scale"], np.float64)
                      [tok if ref["output_scale"].shape[0] != R else slice(None)], 128, axis=1)
    ds = np.repeat(dv.reshape(R, C // 128, 128).max(-1) / 448.0, 128, axis=1)
    lo = codecs.e4m3_decode(codecs.e4m3_encode_sat(np.maximum(v - dv, 0) / (s_ref + ds)))
    hi = codecs.e4m3_decode(codecs.e4m3_encode_sat(np.minimum((v + dv) / np.maximum(s_ref - ds, 1e-300),
                                                              448.0)))
    mid = codecs.e4m3_decode(codecs.e4m3_encode_sat(np.minimum(v / s_ref, 448.0)))
    slack = np.maximum(np.abs(hi * (s_ref + ds) - mid * s_ref), np.abs(mid * s_ref - lo * (s_ref - ds)))
    return allow + slack, slack
