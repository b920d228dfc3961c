"""Pins of the oracle's whole-layer composition, oracle.forward.

Every end-to-end GPU test uses oracle.forward as its reference, so how it
chains the pinned stages is pinned here, three ways:

  * against an independent dense brute force written with torch float64
    (every expert on every token, then masked by the routing), which takes
    the readings of the pages from the pages, not from the oracle:
      - with the router weight on the input (top-1), the weight goes on the
        input *instead of* the output ("Fused MoE Kernel Features", backend
        section), so finalize weights that row by 1;
      - the shared expert's row is added with weight 1 to the weighted top-k
        sum, on the unweighted input, and the residual after it, all before
        RMSNorm ("[flashinfer] MoE Finalize + AllReduce fusion",
        introduction);
  * against the stages chained by hand, bit for bit, on every parity case;
  * by planted mistakes: each one is put into the oracle (on the CPU) and
    one of the checks above must fail on it.
"""

import inspect

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.moe as om
from oracle import codecs
from workloads import PARITY_CASES, make_layer_inputs, to_numpy_bits

CASES = {s.name: s for s in PARITY_CASES}
WKEYS = ("w13", "w13_scale", "w2", "w2_scale", "shared_w13", "shared_w13_scale", "shared_w2",
         "shared_w2_scale")


def _host_w(d):
    return {k: to_numpy_bits(d[k]) for k in WKEYS if d.get(k) is not None}


def _oracle_forward(spec, d, mode="exact", tokens=None):
    return oracle.forward(to_numpy_bits(d["x"]), d["logits"].numpy(), _host_w(d), spec.top_k,
                          spec.scoring, spec.renormalize, 16, spec.apply_router_weight_on_input,
                          spec.quant, spec.activation, mode, to_numpy_bits(d.get("residual")),
                          to_numpy_bits(d.get("gamma")), spec.eps, spec.out_quant, tokens=tokens)


# ---------------------------------------------------------------- brute force
def _torch_weight(codes, scale):
    """[.., N, K] weight -> float64: bf16 values, or E4M3 codes times their
    128x128 block scales (torch's own float8_e4m3fn decode)."""
    if scale is None:
        return codes.double()
    v = codes.view(torch.float8_e4m3fn).double()
    s = scale.double().repeat_interleave(128, dim=-2).repeat_interleave(128, dim=-1)
    return v * s[..., :v.shape[-2], :v.shape[-1]]


def _torch_quant_g128(a32):
    """G(128) E4M3 quantisation in torch: s = max(amax, 1e-10)/448 (float32),
    code = torch's float8_e4m3fn cast of a/s; returns the dequantised float64."""
    T, H = a32.shape
    g = a32.reshape(T, H // 128, 128)
    s = torch.clamp(g.abs().amax(-1, keepdim=True), min=1e-10) / 448.0
    q = (g / s).to(torch.float8_e4m3fn)
    return (q.double() * s.double()).reshape(T, H)


def _bf16_round(v64):
    return torch.from_numpy(codecs.bf16_bits_to_f64(codecs.f64_to_bf16_bits(v64.numpy())))


def _act(name, h, inter):
    fn = (lambda v: v * torch.sigmoid(v)) if name.startswith("silu") else \
        (lambda v: 0.5 * v * (1.0 + torch.erf(v / np.sqrt(2.0))))
    if name in ("silu", "gelu"):
        return fn(h[..., :inter]) * h[..., inter:]
    return fn(h)


def dense_layer(spec, d):
    """The layer with every expert run densely on every token (exact mode:
    intermediates in float64), then selected by the routing.  Returns the
    output decoded to float64 [T, H] (bf16 output only)."""
    assert spec.quant in ("none", "fp8") and spec.out_quant == "none"
    x = d["x"]
    T, H = x.shape
    k = spec.top_k
    lg = d["logits"].double()
    top = torch.topk(lg, k, dim=1, sorted=True)
    assert not (top.values[:, :-1] == top.values[:, 1:]).any(), "tied logits: pick another case"
    ids = top.indices
    p = torch.softmax(lg, dim=1) if spec.scoring == "softmax" else torch.sigmoid(lg)
    w = p.gather(1, ids)
    if spec.renormalize:
        w = w / w.sum(dim=1, keepdim=True)
    w32 = w.float()
    # prepare: top-1 weight on the input (bf16 product), then the quantiser
    xin = x * w32.bfloat16() if spec.apply_router_weight_on_input else x

    def quant(a_bf16):
        return _torch_quant_g128(a_bf16.float()) if spec.quant == "fp8" else a_bf16.double()

    W13 = _torch_weight(d["w13"], d.get("w13_scale"))
    W2 = _torch_weight(d["w2"], d.get("w2_scale"))
    I = W2.shape[-1]
    h = torch.einsum("th,erh->ter", quant(xin), W13)
    y_all = torch.einsum("tei,ehi->teh", _act(spec.activation, h, I), W2)     # [T, E, H]
    y = _bf16_round(y_all[torch.arange(T)[:, None], ids])                      # [T, k, H]
    wt = torch.ones_like(w) if spec.apply_router_weight_on_input else w32.double()
    acc = torch.zeros(T, H, dtype=torch.float64)
    for j in range(k):
        acc = acc + wt[:, j:j + 1] * y[:, j]
    if d.get("shared_w13") is not None:
        S13 = _torch_weight(d["shared_w13"], d.get("shared_w13_scale"))
        S2 = _torch_weight(d["shared_w2"], d.get("shared_w2_scale"))
        hs = quant(x) @ S13.T                                   # the unweighted input
        acc = acc + _bf16_round(_act(spec.activation, hs, S2.shape[-1]) @ S2.T)
    if d.get("residual") is not None:
        acc = acc + d["residual"].double()
    if d.get("gamma") is not None:
        acc = F.rms_norm(acc, (H,), d["gamma"].double(), eps=spec.eps)
    return _bf16_round(acc).numpy()


def _matches_dense(spec, d, ref):
    """True when oracle.forward's output (exact mode) equals the brute force:
    at least 99.9 % of elements bit-identical, the rest within one bf16
    step (two float64 summation orders may round a value at a bf16 midpoint
    differently)."""
    dense = dense_layer(spec, d)
    got = codecs.bf16_bits_to_f64(ref["output"])
    same = float((got == dense).mean())
    close = np.all(np.abs(got - dense) <= 2.0 ** -7 * np.abs(dense) + 1e-30)
    return same >= 0.999 and bool(close), same


DENSE_CASES = ["tiny", "mixtral_mini", "llama4_mini", "llama4_mini_silu_no_mul",
               "finalize_fused_mini", "gelu_mini", "deepseek_mini"]


@pytest.mark.parametrize("name", DENSE_CASES)
def test_forward_equals_dense_brute_force(name):
    spec = CASES[name]
    d = make_layer_inputs(spec)
    ok, same = _matches_dense(spec, d, _oracle_forward(spec, d))
    assert ok, f"{name}: oracle.forward differs from the dense brute force ({same:.4f} identical)"


# ----------------------------------------------------------- stages by hand
def _chain_by_hand(spec, d, mode):
    """route -> prepare -> experts (shared expert on the unweighted input) ->
    finalize (weight 1 on the top-1 row when it went on the input)."""
    hw = _host_w(d)
    x = to_numpy_bits(d["x"])
    ids, tw = oracle.route(d["logits"].numpy(), spec.top_k, spec.scoring, spec.renormalize)
    a1q, a1s = oracle.prepare(x, tw, spec.apply_router_weight_on_input, spec.quant)
    shared = None
    if "shared_w13" in hw:
        sa, ss = oracle.prepare(x, None, False, spec.quant)
        shared = dict(a=sa, a_scale=ss, w13=hw["shared_w13"], w13_scale=hw.get("shared_w13_scale"),
                      w2=hw["shared_w2"], w2_scale=hw.get("shared_w2_scale"))
    feo, sh = oracle.experts(a1q, a1s, ids, hw["w13"], hw.get("w13_scale"), hw["w2"],
                             hw.get("w2_scale"), spec.activation, mode, shared)
    return oracle.finalize(feo, tw, spec.apply_router_weight_on_input, sh,
                           to_numpy_bits(d.get("residual")), to_numpy_bits(d.get("gamma")),
                           spec.eps, spec.out_quant)


@pytest.mark.parametrize("spec", PARITY_CASES, ids=lambda s: s.name)
def test_forward_equals_stages_chained_by_hand(spec):
    d = make_layer_inputs(spec)
    for mode in ("exact", "mirrored"):
        ref = _oracle_forward(spec, d, mode)
        out, out_s, res = _chain_by_hand(spec, d, mode)
        np.testing.assert_array_equal(ref["output"], out, err_msg=f"{spec.name} {mode}")
        if out_s is not None:
            np.testing.assert_array_equal(ref["output_scale"], out_s)
        np.testing.assert_array_equal(ref["residual_out"], res)


@pytest.mark.parametrize("name", ["fp8_tensor_mini", "deepseek_mini", "llama4_mini",
                                  "fp8_out_mini"])
def test_forward_token_subset_is_a_restriction(name):
    """forward(tokens=S) gives the rows of S of the full forward: tokens are
    independent, except that a per-tensor scale is taken over all tokens.
    The full-size GPU tests rely on this to sample tokens."""
    spec = CASES[name]
    d = make_layer_inputs(spec)
    sub = np.array([0, 3, 7, spec.T // 2, spec.T - 1])
    full = _oracle_forward(spec, d, "mirrored")
    part = _oracle_forward(spec, d, "mirrored", tokens=sub)
    np.testing.assert_array_equal(part["output"], full["output"][sub])
    if full["output_scale"] is not None:
        np.testing.assert_array_equal(part["output_scale"], full["output_scale"][sub])


# ------------------------------------------------------------ planted mistakes
def _mutant_forward(old, new):
    """oracle.forward with one source fragment replaced (the fragment must
    exist, so the planted mistake tracks the code it mutates)."""
    src = inspect.getsource(om.forward)
    assert src.count(old) == 1, f"fragment not found once in oracle.forward: {old!r}"
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), "<mutant forward>", "exec"), ns)
    return ns["forward"]


def _run_mutant(monkeypatch, spec, d, forward_fn=None, finalize_fn=None, experts_fn=None):
    if forward_fn is not None:
        monkeypatch.setattr(oracle, "forward", forward_fn)
    if finalize_fn is not None:
        monkeypatch.setattr(om, "finalize", finalize_fn)
    if experts_fn is not None:
        monkeypatch.setattr(om, "experts", experts_fn)
    return _oracle_forward(spec, d)


def test_planted_shared_expert_on_weighted_input_is_caught(monkeypatch):
    """(a) the shared expert fed the router-weighted input under
    weight-on-input."""
    spec = CASES["llama4_mini"]
    d = make_layer_inputs(spec)
    mut = _mutant_forward("sa, ss = prep(None)", "sa, ss = a1q, a1q_scale")
    ref = _run_mutant(monkeypatch, spec, d, forward_fn=mut)
    assert not _matches_dense(spec, d, ref)[0]
    out, _, _ = _chain_by_hand(spec, d, "exact")
    assert not np.array_equal(ref["output"], out)


def test_planted_weight_on_input_and_output_is_caught(monkeypatch):
    """(b) finalize weights the top-1 row by w although w already went on
    the input (w' = w instead of 1)."""
    spec = CASES["llama4_mini"]
    d = make_layer_inputs(spec)
    real = om.finalize

    def finalize_reweights(feo, tw, woi, *a, **kw):
        return real(feo, tw, False, *a, **kw)
    ref = _run_mutant(monkeypatch, spec, d, finalize_fn=finalize_reweights)
    assert not _matches_dense(spec, d, ref)[0]


def test_planted_per_tensor_scale_over_subset_is_caught():
    """(c) the per-tensor scale taken over the sampled tokens only."""
    spec = CASES["fp8_tensor_mini"]
    d = make_layer_inputs(spec)
    mut = _mutant_forward('if quant == "fp8_tensor":', "if False:")
    sub = np.array([0, 3, 7, spec.T // 2, spec.T - 1])
    args = (to_numpy_bits(d["x"]), d["logits"].numpy(), _host_w(d), spec.top_k, spec.scoring,
            spec.renormalize, 16, spec.apply_router_weight_on_input, spec.quant, spec.activation,
            "mirrored")
    full = oracle.forward(*args)
    part = mut(*args, tokens=sub)
    assert not np.array_equal(part["output"], full["output"][sub])


def test_planted_shared_and_residual_after_rmsnorm_is_caught(monkeypatch):
    """(d) the shared row and the residual added after RMSNorm instead of
    before it."""
    spec = CASES["finalize_fused_mini"]
    d = make_layer_inputs(spec)
    real = om.finalize

    def finalize_late_adds(feo, tw, woi, shared=None, residual=None, gamma=None, eps=1e-6,
                           out_quant="none", tokens=None):
        out, s, res = real(feo, tw, woi, None, None, gamma, eps, "none", tokens)
        v = codecs.bf16_bits_to_f64(out)
        tok = np.arange(feo.shape[0]) if tokens is None else tokens
        for extra in (shared, residual):
            if extra is not None:
                v = v + codecs.bf16_bits_to_f64(extra)[tok]
        return codecs.f64_to_bf16_bits(v), s, res
    ref = _run_mutant(monkeypatch, spec, d, finalize_fn=finalize_late_adds)
    assert not _matches_dense(spec, d, ref)[0]


def test_planted_shared_expert_weighted_in_finalize_is_caught(monkeypatch):
    """(e) the shared row scaled by a router weight instead of 1."""
    spec = CASES["finalize_fused_mini"]
    d = make_layer_inputs(spec)
    real = om.finalize

    def finalize_weighted_shared(feo, tw, woi, shared=None, *a, **kw):
        if shared is not None:
            w0 = np.asarray(tw, np.float64)[:, :1]
            shared = codecs.f64_to_bf16_bits(codecs.bf16_bits_to_f64(shared) * w0)
        return real(feo, tw, woi, shared, *a, **kw)
    ref = _run_mutant(monkeypatch, spec, d, finalize_fn=finalize_weighted_shared)
    assert not _matches_dense(spec, d, ref)[0]


def test_planted_slot_dropped_is_caught(monkeypatch):
    """(f) the experts stage losing the last top-k slot of every token."""
    spec = CASES["mixtral_mini"]
    d = make_layer_inputs(spec)
    real = om.experts

    def experts_drop_slot(*a, **kw):
        feo, sh = real(*a, **kw)
        feo = feo.copy()
        feo[:, -1] = 0
        return feo, sh
    ref = _run_mutant(monkeypatch, spec, d, experts_fn=experts_drop_slot)
    assert not _matches_dense(spec, d, ref)[0]
