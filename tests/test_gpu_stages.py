"""GPU parity of the per-stage C entry points (route, prepare, align,
finalize) against the CPU oracle, on the seeded workloads and edge cases.
Integer results (ids, sorted rows, offsets, fp8 codes) are bit-exact;
floating-point results meet the stated tolerances."""

import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs
from workloads import CONFIGS, PARITY_CASES, make_layer_inputs, make_finalize_inputs, to_numpy_bits
from helpers import check_tolerance, f64_of_bf16, f64_of_fp8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _moe():
    import mixture_experts_layer_routing_amd as moe
    return moe


def _announce(name):
    print(f"[case] {name}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ route
def _route_cases():
    cases = []
    for fam in ("tiny", "mixtral", "deepseek_v3", "llama4"):
        for spec in CONFIGS[fam]:
            if spec.activation != "silu":
                continue
            cases.append((spec.name, spec))
    return cases


@pytest.mark.parametrize("name,spec", _route_cases(), ids=[c[0] for c in _route_cases()])
def test_route_matches_oracle_on_config_logits(name, spec):
    _announce(f"route {name}")
    moe = _moe()
    logits = make_layer_inputs(spec, weights=False)["logits"]
    ids, w = moe.moe_route(logits.to(DEV), spec.top_k, spec.scoring, spec.renormalize)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits.numpy(), spec.top_k, spec.scoring, spec.renormalize)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=0, atol=1e-5)


@pytest.mark.parametrize("T,E,k,scoring,renorm", [
    (257, 8, 2, "softmax", True), (100, 1024, 64, "softmax", False), (33, 1, 1, "sigmoid", True),
    (64, 300, 7, "sigmoid", False), (5, 64, 64, "softmax", True), (1000, 16, 1, "softmax", False)])
def test_route_edge_shapes_and_ties(T, E, k, scoring, renorm):
    _announce(f"route T={T} E={E} k={k}")
    moe = _moe()
    g = torch.Generator().manual_seed(T * 7 + E)
    # few distinct values: many exact ties, resolved to the lower expert index
    logits = (torch.randint(-4, 4, (T, E), generator=g).float() * 0.5)
    ids, w = moe.moe_route(logits.to(DEV), k, scoring, renorm)
    torch.cuda.synchronize()
    rid, rw = oracle.route(logits.numpy(), k, scoring, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=0, atol=1e-5)


def test_route_rejects_bad_arguments():
    moe = _moe()
    logits = torch.zeros((4, 8), device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_route(logits, 9)
    with pytest.raises(moe.MoeError):
        moe.moe_route(logits, 0)


# ---------------------------------------------------------------- prepare
@pytest.mark.parametrize("T,H,flag,quant", [
    (16, 128, False, "fp8"), (203, 768, False, "fp8"), (64, 7168, False, "fp8"),
    (157, 640, True, "none"), (128, 5120, True, "none"), (77, 512, True, "fp8"),
    (1, 7168, False, "fp8"), (3, 8, True, "none"),
    (203, 768, False, "fp8_token"), (64, 7168, True, "fp8_token"), (5, 16384, False, "fp8_token"),
    (1, 128, False, "fp8_token"), (203, 768, False, "fp8_tensor"), (77, 5120, True, "fp8_tensor"),
    (4096, 7168, False, "fp8_tensor"), (1, 128, False, "fp8_tensor")])
def test_prepare_bit_exact(T, H, flag, quant):
    _announce(f"prepare T={T} H={H} flag={flag} {quant}")
    moe = _moe()
    g = torch.Generator().manual_seed(T + H)
    x = (torch.randn((T, H), generator=g) * torch.rand((T, 1), generator=g) * 10).to(torch.bfloat16)
    x[0, :8] = 0.0                                   # a zero run (zero group when H == 8)
    tw = torch.rand((T, 1), generator=g) if flag else None
    q, s = moe.moe_prepare(x.to(DEV), None if tw is None else tw.to(DEV),
                           apply_router_weight_on_input=flag, quant=quant)
    torch.cuda.synchronize()
    rq, rs = oracle.prepare(to_numpy_bits(x), None if tw is None else tw.numpy(), flag, quant)
    np.testing.assert_array_equal(to_numpy_bits(q), rq)
    if quant.startswith("fp8"):
        np.testing.assert_array_equal(s.cpu().numpy().reshape(rs.shape), rs)


def test_prepare_zero_group_and_constant_group():
    moe = _moe()
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    x[1, :128] = -3.0
    x[1, 128:] = 448.0
    q, s = moe.moe_prepare(x.to(DEV), quant="fp8")
    torch.cuda.synchronize()
    rq, rs = oracle.prepare(to_numpy_bits(x), None, False, "fp8")
    np.testing.assert_array_equal(to_numpy_bits(q), rq)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)


def test_prepare_rejects_weight_on_input_with_top_k_2():
    moe = _moe()
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_prepare(x, torch.ones((4, 2), device=DEV), apply_router_weight_on_input=True)


# ------------------------------------------------------------------ align
def _align_compare(ids_cpu, E, BM):
    moe = _moe()
    out = moe.moe_align(ids_cpu.to(DEV), E, BM)
    torch.cuda.synchronize()
    ref = oracle.align(ids_cpu.numpy(), E, BM)
    for k in ("expert_counts", "expert_offsets", "sorted_token_ids", "block_expert_ids",
              "num_tokens_post_padded"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), ref[k], err_msg=k)


def _align_config_cases():
    out = []
    for fam in ("tiny", "mixtral", "deepseek_v3", "llama4"):
        for spec in CONFIGS[fam]:
            if spec.activation != "silu":
                continue
            out.append(spec)
    return out


@pytest.mark.parametrize("spec", _align_config_cases(), ids=lambda s: s.name)
@pytest.mark.parametrize("BM", [16, 64, 128])
def test_align_bit_exact_on_config_routing(spec, BM):
    _announce(f"align {spec.name} BM={BM}")
    logits = make_layer_inputs(spec, weights=False)["logits"]
    rid, _ = oracle.route(logits.numpy(), spec.top_k, spec.scoring, spec.renormalize)
    _align_compare(torch.from_numpy(rid), spec.E, BM)


@pytest.mark.parametrize("T,k,E,BM,pattern", [
    (5000, 1, 8, 16, "one_expert"), (9000, 8, 256, 32, "hot"), (4096, 1, 16, 256, "random"),
    (4097, 1, 16, 64, "random"), (1, 2, 8, 16, "random"), (0, 2, 8, 16, "random"),
    (20000, 4, 1024, 128, "random"), (3000, 2, 3, 16, "empty"),
    (4096, 8, 256, 64, "random"), (4097, 8, 256, 64, "hot")])
def test_align_adversarial(T, k, E, BM, pattern):
    _announce(f"align adversarial T={T} k={k} E={E} BM={BM} {pattern}")
    g = torch.Generator().manual_seed(T + E)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]) if T else \
        torch.zeros((0, k), dtype=torch.long)
    if pattern == "one_expert":
        ids[:] = 5
    elif pattern == "hot":
        ids[: T // 2, 0] = 7
        ids[: T // 2, 1:] = torch.where(ids[: T // 2, 1:] == 7, 8, ids[: T // 2, 1:])
    elif pattern == "empty":
        ids[:] = torch.where(ids == 1, 0, ids)   # expert 1 never chosen
        ids[:, 1] = 2
        ids[:, 0] = 0
    _align_compare(ids.to(torch.int32).contiguous(), E, BM)


@pytest.mark.parametrize("T,k,E,BM", [(20000, 8, 256, 128), (200000, 8, 256, 128),
                                      (600000, 8, 64, 64), (2100000, 2, 8, 256),
                                      (2100001, 8, 256, 128), (600000, 4, 1024, 128),
                                      (300000, 1, 3, 16)])
def test_align_multi_tile_sizes(T, k, E, BM):
    """Every tile size from the 2048-id minimum to the 8192-id maximum (over
    2^23 ids), tile counts that are not a multiple of the 8 XCDs, the column
    scan over more tiles than one pass of its workgroup, E up to 1024 (the
    larger LDS sizing of the scatter), a ragged last tile."""
    _announce(f"align large T={T} k={k} E={E} BM={BM}")
    g = torch.Generator().manual_seed(T + E)
    ids = torch.rand((T, E), generator=g).argsort(dim=1)[:, :k].to(torch.int32).contiguous()
    _align_compare(ids, E, BM)


@pytest.mark.parametrize("T,k,E,BM", [(20000, 8, 256, 128), (600000, 8, 64, 64),
                                      (300000, 1, 3, 16), (4097, 8, 256, 64)])
def test_align_tiled_path_where_the_resident_one_applies(T, k, E, BM, monkeypatch):
    """The three-launch tiled path, forced (MOE_ALIGN_RESIDENT=0) on sizes
    the one-launch resident path takes by default: both are bit-exact."""
    _announce(f"align tiled T={T} k={k} E={E} BM={BM}")
    monkeypatch.setenv("MOE_ALIGN_RESIDENT", "0")
    g = torch.Generator().manual_seed(T + E + 1)
    ids = torch.randint(0, E, (T, k), generator=g, dtype=torch.int32)
    _align_compare(ids, E, BM)


@pytest.mark.parametrize("n,E,BM", [(1 << 24, 256, 128), (1 << 24, 8, 256),
                                    ((1 << 24) - 1000, 16, 32), (204 * 1024 + 77, 256, 16),
                                    (3 * 65536 + 5, 9, 64)])
def test_align_resident_grid_shapes(n, E, BM):
    """The resident path at its capacity (2^24 ids: 256 workgroups of 65536
    ids, 64 per lane) and below it: a ragged last tile, a grid that is not a
    multiple of the 8 XCDs, the ballot rank (E <= 8) and the table rank."""
    _announce(f"align resident n={n} E={E} BM={BM}")
    g = torch.Generator().manual_seed(n % 9973 + E)
    ids = torch.randint(0, E, (n, 1), generator=g, dtype=torch.int32)
    _align_compare(ids, E, BM)


def test_align_is_deterministic_across_runs():
    moe = _moe()
    g = torch.Generator().manual_seed(3)
    ids = torch.randint(0, 64, (30000, 2), generator=g, dtype=torch.int32).to(DEV)
    a = moe.moe_align(ids, 64, 16)
    b = moe.moe_align(ids, 64, 16)
    torch.cuda.synchronize()
    assert torch.equal(a["sorted_token_ids"], b["sorted_token_ids"])


# --------------------------------------------------------------- finalize
def _finalize_case(spec, sample=None):
    moe = _moe()
    d = make_finalize_inputs(spec)
    dd = {k: v.to(DEV) for k, v in d.items()}
    out, scale, res_out = moe.moe_finalize(
        dd["fused_expert_output"], dd["topk_weights"], dd["topk_ids"], False, dd.get("shared"),
        dd.get("residual"), dd.get("gamma"), spec.eps, spec.out_quant, want_residual_out=True)
    torch.cuda.synchronize()
    tok = None if sample is None else np.asarray(sample)
    ro, rs, rres = oracle.finalize(to_numpy_bits(d["fused_expert_output"]), d["topk_weights"].numpy(),
                                   False, to_numpy_bits(d["shared"]), to_numpy_bits(d["residual"]),
                                   to_numpy_bits(d["gamma"]), spec.eps, spec.out_quant, tokens=tok)
    sel = slice(None) if tok is None else tok
    if spec.out_quant == "fp8":
        got = f64_of_fp8(to_numpy_bits(out)[sel], scale.cpu().numpy()[sel])
        ref = f64_of_fp8(ro, rs)
        check_tolerance(got, ref, None, "fp8", spec.name)
        # codes differ by at most one step where the fp32 and fp64 values straddle a rounding edge
        gc = codecs.e4m3_decode(to_numpy_bits(out)[sel])
        rc = codecs.e4m3_decode(ro)
        step = np.maximum(np.abs(rc) * 2.0 ** -3, 2.0 ** -9)
        assert np.all(np.abs(gc - rc) <= step + 1e-12)
        np.testing.assert_allclose(scale.cpu().numpy()[sel], rs, rtol=1e-5)
    else:
        got = f64_of_bf16(to_numpy_bits(out)[sel])
        ref = f64_of_bf16(ro)
        check_tolerance(got, ref, ref, "bf16", spec.name)
    # residual_out = bf16(acc): one bf16 ulp apart at most, plus the fp32-vs-fp64
    # accumulation error where the sum cancels towards zero
    gr = f64_of_bf16(to_numpy_bits(res_out)[sel])
    rr = f64_of_bf16(rres)
    assert np.all(np.abs(gr - rr) <= np.abs(rr) * 2.0 ** -7 + 1e-5)


@pytest.mark.parametrize("spec", CONFIGS["finalize"], ids=lambda s: s.name)
def test_finalize_configs(spec):
    _announce(f"finalize {spec.name}")
    sample = None
    if spec.T > 512:
        rng = np.random.default_rng(spec.T)
        sample = np.sort(rng.choice(spec.T, size=256, replace=False))
        sample[-1] = spec.T - 1
    _finalize_case(spec, sample)


@pytest.mark.parametrize("k,flag,shared,res,gamma", [
    (1, True, True, False, True), (2, False, False, False, False), (8, False, True, True, False),
    (1, False, False, True, True)])
def test_finalize_variants(k, flag, shared, res, gamma):
    _announce(f"finalize variant k={k} flag={flag}")
    moe = _moe()
    T, H = 37, 1024
    g = torch.Generator().manual_seed(k * 10 + flag)
    y = torch.randn((T, k, H), generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn((T, k), generator=g), 1)
    sh = torch.randn((T, H), generator=g).to(torch.bfloat16) if shared else None
    rs = torch.randn((T, H), generator=g).to(torch.bfloat16) if res else None
    gm = (0.5 + torch.rand(H, generator=g)).to(torch.bfloat16) if gamma else None
    dv = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    out, _, _ = moe.moe_finalize(y.to(DEV), w.to(DEV), None, flag, dv(sh), dv(rs), dv(gm), 1e-6)
    torch.cuda.synchronize()
    ro, _, _ = oracle.finalize(to_numpy_bits(y), w.numpy(), flag,
                               None if sh is None else to_numpy_bits(sh),
                               None if rs is None else to_numpy_bits(rs),
                               None if gm is None else to_numpy_bits(gm), 1e-6)
    ref = f64_of_bf16(ro)
    check_tolerance(f64_of_bf16(out), ref, ref, "bf16", "finalize variant")
