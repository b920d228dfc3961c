"""GPU parity of the one-launch layer (moe_forward_monolithic) against the
CPU oracle: reduced decode-sized cases element by element (the bar of the
modular forward: bf16 sums in another order, the z-flip allowance), the
Mixtral family at full size, and the paths that only the one-launch kernel
has (experts holding more than one 16-row group, every routing width,
weight on the input with a shared expert, RMSNorm and fp8 output)."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, PARITY_CASES, make_layer_inputs, to_numpy_bits
from workloads.configs import TINY
from helpers import check_tolerance, output_allowance, f64_of_bf16, f64_of_fp8

pytestmark = pytest.mark.gpu
DEV = "cuda"
WKEYS = ("w13", "w2", "w13_scale", "w2_scale", "shared_w13", "shared_w2", "shared_w13_scale",
         "shared_w2_scale")


def _moe():
    import mixture_experts_layer_routing_amd as moe
    return moe


def _announce(name):
    print(f"[case] {name}", file=sys.stderr, flush=True)


def _case(name, **kw):
    base = TINY if name == "tiny" else next(s for s in PARITY_CASES if s.name == name)
    return dataclasses.replace(base, **kw)


# bf16 weights, T <= 512, T*top_k <= 512
CASES = [
    _case("tiny"),                                                   # T=16, k=2
    _case("mixtral_mini", T=32),                                     # 64 rows over 8 experts
    _case("tiny", T=64, E=2, top_k=1),                               # 32 rows an expert: 2 row groups
    _case("tiny", T=8, E=256, top_k=8, scoring="sigmoid"),          # 64 experts touched
    _case("tiny", T=6, E=1024, top_k=2, renormalize=False),          # 1024-wide routing
    _case("llama4_mini", T=40),                                      # weight on the input + shared
    _case("llama4_mini_silu_no_mul", T=16),
    _case("finalize_fused_mini", T=16),                              # k=4, shared, residual, RMSNorm
    _case("finalize_fused_mini", T=16, out_quant="fp8"),
    _case("gelu_mini", T=16),
    _case("decode_split_mini"),                                      # H = I = 2048, shared
    _case("decode_split_no_mul_mini"),
    _case("shared_dense_mini", T=32),                                # 2 shared row groups
    # up to 512 routed rows: experts with several 16-row groups, 16 shared groups
    _case("llama4_mini"),                                            # T=157, top-1, weight on input
    _case("mixtral_mini", T=200),                                    # 400 rows over 8 experts
    _case("tiny", T=64, E=256, top_k=8, scoring="sigmoid"),          # 512 rows
    _case("shared_dense_mini", T=256),                               # 512 rows, residual, RMSNorm
    # fp8 weights (E4M3, 128 x 128 blocks; x and z quantised to G(128) in the kernel)
    _case("decode_split_fp8_mini"),                                  # T=3, k=4, shared, split K
    _case("deepseek_mini", T=64),                                    # 512 rows, sigmoid, hot experts
    _case("fp8_out_mini"),                                           # T=77, k=4, RMSNorm, fp8 out
    _case("deepseek_mini", T=5, activation="silu_no_mul"),
]


def _weights(moe, d, quant="none"):
    return moe.make_weights(*(d.get(k) for k in ("w13", "w2", "w13_scale", "w2_scale",
                                                 "shared_w13", "shared_w2", "shared_w13_scale",
                                                 "shared_w2_scale")),
                            quant=None if quant == "none" else quant)


def _run(moe, spec, dd, w):
    out, scale, _ = moe.moe_forward_monolithic(
        dd["x"], dd["logits"], w, spec.top_k, spec.scoring, spec.renormalize,
        spec.apply_router_weight_on_input, spec.activation, dd.get("residual"), dd.get("gamma"),
        spec.eps, spec.out_quant)
    torch.cuda.synchronize()
    return out, scale


def _f64(spec, out, scale):
    if spec.out_quant == "fp8":
        return f64_of_fp8(to_numpy_bits(out), scale.cpu().numpy())
    return f64_of_bf16(to_numpy_bits(out))


def _ref64(spec, r):
    if spec.out_quant == "fp8":
        return f64_of_fp8(r["output"], r["output_scale"])
    return f64_of_bf16(r["output"])


def _check_against_oracle(spec, d, out, scale, label):
    hw = {k: to_numpy_bits(d[k]) for k in WKEYS if d.get(k) is not None}
    refs = {mode: oracle.forward(to_numpy_bits(d["x"]), d["logits"].cpu().numpy(), hw, spec.top_k,
                                 spec.scoring, spec.renormalize, 16,
                                 spec.apply_router_weight_on_input, spec.quant, spec.activation,
                                 mode, to_numpy_bits(d.get("residual")),
                                 to_numpy_bits(d.get("gamma")), spec.eps, spec.out_quant)
            for mode in ("exact", "mirrored")}
    allowance, slack = output_allowance(spec, refs["mirrored"], d, hw)
    path = "fp8" if (spec.quant != "none" or spec.out_quant == "fp8") else "bf16"
    check_tolerance(_f64(spec, out, scale), _ref64(spec, refs["exact"]),
                    _ref64(spec, refs["mirrored"]), path, label,
                    min_identical=0.9 if path == "bf16" else None,
                    allowance=allowance, maxnorm_slack=slack)


@pytest.mark.parametrize("spec", CASES, ids=lambda s: f"{s.name}@T{s.T}E{s.E}k{s.top_k}"
                         + ("+fp8out" if s.out_quant == "fp8" else ""))
def test_monolithic_matches_the_oracle(spec):
    _announce(f"monolithic {spec.name} T={spec.T} E={spec.E} k={spec.top_k}")
    moe = _moe()
    d = make_layer_inputs(spec)
    dd = {k: v.to(DEV) for k, v in d.items()}
    w = _weights(moe, dd, spec.quant)
    out, scale = _run(moe, spec, dd, w)
    _check_against_oracle(spec, d, out, scale, f"monolithic {spec.name}")
    # a fixed summation order: a second launch gives the same bits
    out2, scale2 = _run(moe, spec, dd, w)
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    if scale is not None:
        assert torch.equal(scale, scale2)


def test_monolithic_residual_out_and_modular_agreement():
    """residual_out is bf16 of the pre-norm sum, as the modular forward's;
    both layers agree within the bf16 bar of either against the oracle."""
    _announce("monolithic residual_out")
    moe = _moe()
    spec = _case("finalize_fused_mini", T=16)
    d = make_layer_inputs(spec)
    dd = {k: v.to(DEV) for k, v in d.items()}
    w = _weights(moe, dd)
    r_mono = torch.empty_like(dd["x"])
    r_mod = torch.empty_like(dd["x"])
    a, _, _ = moe.moe_forward_monolithic(dd["x"], dd["logits"], w, spec.top_k, spec.scoring,
                                         spec.renormalize, False, spec.activation,
                                         dd["residual"], dd["gamma"], spec.eps,
                                         residual_out=r_mono)
    b, _, _ = moe.moe_forward(dd["x"], dd["logits"], w, spec.top_k, spec.scoring,
                              spec.renormalize, False, spec.activation, 0, dd["residual"],
                              dd["gamma"], spec.eps, residual_out=r_mod)
    torch.cuda.synchronize()
    ra, rb = f64_of_bf16(to_numpy_bits(r_mono)), f64_of_bf16(to_numpy_bits(r_mod))
    scale = np.abs(rb).max()
    assert np.abs(ra - rb).max() <= 2e-2 * scale
    oa, ob = f64_of_bf16(to_numpy_bits(a)), f64_of_bf16(to_numpy_bits(b))
    assert np.abs(oa - ob).max() <= 2e-2 * np.abs(ob).max()


def test_monolithic_mixtral_full_size():
    """Mixtral's decode shapes at full size (H=4096, I=14336, E=8, top-2):
    T = 1 and 8, every token against the oracle."""
    moe = _moe()
    fam = CONFIGS["mixtral"]
    d0 = None
    w = None
    for T in (1, 8):
        spec = dataclasses.replace(fam[0], T=T)
        _announce(f"monolithic full mixtral T={T}")
        if d0 is None:
            d0 = make_layer_inputs(spec, device=DEV)
            w = _weights(moe, d0)
            hw = {k: to_numpy_bits(d0[k]) for k in WKEYS if d0.get(k) is not None}
        d = make_layer_inputs(spec, device=DEV, weights=False)
        d.update({k: d0[k] for k in WKEYS if d0.get(k) is not None})
        out, scale = _run(moe, spec, d, w)
        refs = {mode: oracle.forward(to_numpy_bits(d["x"]), d["logits"].cpu().numpy(), hw,
                                     spec.top_k, spec.scoring, spec.renormalize, 16, False, "none",
                                     spec.activation, mode)
                for mode in ("exact", "mirrored")}
        allowance, slack = output_allowance(spec, refs["mirrored"], d, hw)
        check_tolerance(_f64(spec, out, scale), _ref64(spec, refs["exact"]),
                        _ref64(spec, refs["mirrored"]), "bf16", f"monolithic mixtral T={T}",
                        min_identical=0.9, allowance=allowance, maxnorm_slack=slack)


def test_monolithic_llama4_full_size():
    """Llama-4 at T=128 (H=5120, I=8192, E=16, top-1 with the weight on the
    input, an 8192-wide shared expert): 64 sampled tokens against the
    oracle."""
    _announce("monolithic full llama4 T=128")
    moe = _moe()
    spec = CONFIGS["llama4"][0]
    assert spec.T == 128
    d = make_layer_inputs(spec, device=DEV)
    w = _weights(moe, d)
    out, scale = _run(moe, spec, d, w)
    hw = {k: to_numpy_bits(d[k]) for k in WKEYS if d.get(k) is not None}
    rng = np.random.default_rng(128)
    tok = np.unique(np.concatenate([[0, spec.T - 1], rng.choice(spec.T, 62, replace=False)]))
    refs = {mode: oracle.forward(to_numpy_bits(d["x"]), d["logits"].cpu().numpy(), hw, spec.top_k,
                                 spec.scoring, spec.renormalize, 16,
                                 spec.apply_router_weight_on_input, "none", spec.activation, mode,
                                 tokens=tok)
            for mode in ("exact", "mirrored")}
    allowance, slack = output_allowance(spec, refs["mirrored"], d, hw)
    got = f64_of_bf16(to_numpy_bits(out)[tok])
    check_tolerance(got, _ref64(spec, refs["exact"]), _ref64(spec, refs["mirrored"]), "bf16",
                    "monolithic llama4 T=128", min_identical=0.9, allowance=allowance,
                    maxnorm_slack=slack)
    del d, w


def test_monolithic_deepseek_full_size():
    """DeepSeek-V3 fp8 at T=64 (H=7168, I=2048, E=256, top-8, a 2048-wide
    shared expert): 512 routed rows over ~220 experts.  Four tokens against
    the mirrored oracle at the max-norm bar the full-size modular test uses
    for fp8 (the derived per-element fp8 bound walks every touched expert in
    float64), and every token against the modular forward."""
    _announce("monolithic full deepseek_v3 T=64")
    moe = _moe()
    spec = CONFIGS["deepseek_v3"][0]
    assert spec.T == 64
    d = make_layer_inputs(spec, device=DEV)
    w = _weights(moe, d, spec.quant)
    out, scale = _run(moe, spec, d, w)
    ref_out, _, _ = moe.moe_forward(d["x"], d["logits"], w, spec.top_k, spec.scoring,
                                    spec.renormalize, False, spec.activation)
    torch.cuda.synchronize()
    a, b = f64_of_bf16(to_numpy_bits(out)), f64_of_bf16(to_numpy_bits(ref_out))
    assert np.abs(a - b).max() <= 0.06 * np.abs(b).max()
    hw = {k: to_numpy_bits(d[k]) for k in WKEYS if d.get(k) is not None}
    tok = np.array([0, 21, 42, spec.T - 1])
    ref = oracle.forward(to_numpy_bits(d["x"]), d["logits"].cpu().numpy(), hw, spec.top_k,
                         spec.scoring, spec.renormalize, 16, False, spec.quant, spec.activation,
                         "mirrored", tokens=tok)
    check_tolerance(a[tok], None, f64_of_bf16(ref["output"]), "fp8", "monolithic deepseek T=64",
                    elementwise=False)
    del d, w


def test_monolithic_rejects_what_it_does_not_cover():
    _announce("monolithic limits")
    moe = _moe()
    spec = _case("tiny")
    d = {k: v.to(DEV) for k, v in make_layer_inputs(spec).items()}
    w = _weights(moe, d)
    # T * top_k above 512 rows
    x = torch.zeros((257, spec.H), dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros((257, spec.E), dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.moe_forward_monolithic(x, lg, w, spec.top_k)
    # fp8 with per-token activation scales, and fp8 with the weight on the input
    fspec = _case("fp8_token_mini", T=8)
    fd = {k: v.to(DEV) for k, v in make_layer_inputs(fspec).items()}
    fw = _weights(moe, fd, fspec.quant)
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.moe_forward_monolithic(fd["x"], fd["logits"], fw, fspec.top_k)
    gspec = _case("gelu_no_mul_fp8_mini", T=8)
    gd = {k: v.to(DEV) for k, v in make_layer_inputs(gspec).items()}
    gw = _weights(moe, gd, gspec.quant)
    with pytest.raises(moe.MoeError, match="UNSUPPORTED"):
        moe.moe_forward_monolithic(gd["x"], gd["logits"], gw, gspec.top_k, "softmax", False, True,
                                   gspec.activation)
