"""Seeded input generation (random draws and storage casts only)."""

import numpy as np
import torch

from .configs import WorkloadSpec, FinalizeSpec

# fp8 weights: codes are drawn as N(0,1) * FP8_SPREAD clipped to +-448 and
# cast to E4M3 (about 4.5 sigma reaches 448, the top of the format), and every 128x128 block gets
# a float32 scale std / FP8_SPREAD * U(0.75, 1.25), so that code * scale has
# roughly the N(0, 1/sqrt(fan_in)) spread of the bf16 weights.
FP8_SPREAD = 448.0 / 4.5
BLOCK = 128


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)


def _bf16_matrix_stack(n, rows, cols, std, g, device):
    out = torch.empty((n, rows, cols), dtype=torch.bfloat16, device=device)
    for e in range(n):                       # experts drawn in index order
        out[e] = _randn((rows, cols), g, device, std).to(torch.bfloat16)
    return out


def _fp8_matrix_stack(n, rows, cols, std, g, device):
    codes = torch.empty((n, rows, cols), dtype=torch.uint8, device=device)
    scales = torch.empty((n, -(-rows // BLOCK), -(-cols // BLOCK)), dtype=torch.float32,
                         device=device)
    for e in range(n):
        v = _randn((rows, cols), g, device, FP8_SPREAD).clamp_(-448.0, 448.0)
        codes[e] = v.to(torch.float8_e4m3fn).view(torch.uint8)
        u = torch.rand(scales.shape[1:], generator=g, device=device, dtype=torch.float32)
        scales[e] = (0.75 + 0.5 * u) * (std / FP8_SPREAD)
    return codes, scales


def hot_expert_tokens(spec: WorkloadSpec, device="cpu"):
    """(hot expert ids, forced token ids) for the hot-expert recipe: a seeded
    choice of ``hot_experts`` experts and round(hot_fraction * T) tokens."""
    g = _gen(1000 * spec.config + 9, "cpu")
    hot = torch.randperm(spec.E, generator=g)[:spec.hot_experts]
    n_forced = int(round(spec.hot_fraction * spec.T))
    toks = torch.randperm(spec.T, generator=g)[:n_forced] if spec.T else torch.zeros(0, dtype=torch.long)
    return hot.to(device), toks.to(device)


def make_layer_inputs(spec: WorkloadSpec, device="cpu", weights=True):
    """All inputs of one layer call, as torch tensors on ``device``:
    x bf16 [T,H]; logits f32 [T,E]; w13 [E,R,H] (R = 2I for the gated
    activations silu and gelu, I for silu_no_mul and gelu_no_mul) and w2 [E,H,I], bf16 or fp8 codes (uint8) with float32
    128x128 block scales w13_scale/w2_scale; optional shared_w13/shared_w2
    (+scales); optional residual bf16 [T,H] and gamma bf16 [H]."""
    base = 1000 * spec.config
    T, H, I, E = spec.T, spec.H, spec.I, spec.E
    out = {}
    g = _gen(base + 1, device)
    logits = _randn((T, E), g, device, spec.logit_std)
    if spec.hot_experts and T:
        hot, toks = hot_expert_tokens(spec, device)
        rows = toks[:, None].expand(-1, hot.numel())
        cols = hot[None, :].expand(toks.numel(), -1)
        logits[rows, cols] += spec.hot_boost
    out["logits"] = logits
    g = _gen(base + 2, device)
    out["x"] = _randn((T, H), g, device).to(torch.bfloat16)
    if weights:
        R = I if spec.activation.endswith("_no_mul") else 2 * I
        mats = [("w13", 3, E, R, H, H), ("w2", 4, E, H, I, I)]
        if spec.shared_I:
            Rs = spec.shared_I if spec.activation.endswith("_no_mul") else 2 * spec.shared_I
            mats += [("shared_w13", 5, 1, Rs, H, H), ("shared_w2", 6, 1, H, spec.shared_I, spec.shared_I)]
        for name, idx, n, rows, cols, fan_in in mats:
            g = _gen(base + idx, device)
            std = 1.0 / np.sqrt(fan_in)
            if spec.quant.startswith("fp8"):
                c, s = _fp8_matrix_stack(n, rows, cols, std, g, device)
                out[name], out[name + "_scale"] = c, s
            else:
                out[name] = _bf16_matrix_stack(n, rows, cols, std, g, device)
            if name.startswith("shared"):
                out[name] = out[name][0]
                if name + "_scale" in out:
                    out[name + "_scale"] = out[name + "_scale"][0]
    if spec.residual:
        g = _gen(base + 7, device)
        out["residual"] = _randn((T, H), g, device).to(torch.bfloat16)
    if spec.rmsnorm:
        g = _gen(base + 8, device)
        out["gamma"] = (0.5 + torch.rand((H,), generator=g, device=device)).to(torch.bfloat16)
    return out


def make_batched_inputs(spec: WorkloadSpec, M, device="cpu"):
    """Inputs of the experts stage on the batched format: ``a`` bf16
    [E, M, H] ~N(0,1), every row drawn (rows past an expert's count too,
    which the stage must ignore); ``expert_num_tokens`` int32 [E] ~U{0..M},
    then expert 0 set empty and expert E-1 full when E > 1; plus the
    weights of make_layer_inputs for ``spec``."""
    base = 1000 * spec.config
    out = make_layer_inputs(spec.with_T(0), device)
    del out["x"], out["logits"]
    g = _gen(base + 13, device)
    out["a"] = _randn((spec.E, M, spec.H), g, device).to(torch.bfloat16)
    g = _gen(base + 14, "cpu")
    counts = torch.randint(0, M + 1, (spec.E,), generator=g, dtype=torch.int32)
    if spec.E > 1:
        counts[0] = 0
        counts[-1] = M
    out["expert_num_tokens"] = counts.to(device)
    return out


def make_finalize_inputs(spec: FinalizeSpec, device="cpu"):
    """Inputs of the finalize fusion: fused_expert_output bf16 [T,k,H] ~N(0,1);
    topk_weights f32 [T,k] = softmax of N(0,1) draws (drawn and normalised
    here with torch in float64: an input recipe, not the layer's routing);
    topk_ids int32 [T,k] distinct in [0,256); shared and residual bf16 [T,H]
    ~N(0,1); gamma bf16 [H] ~U(0.5,1.5)."""
    base = 1000 * spec.config
    T, k, H = spec.T, spec.top_k, spec.H
    out = {}
    g = _gen(base + 10, device)
    out["fused_expert_output"] = _randn((T, k, H), g, device).to(torch.bfloat16)
    g = _gen(base + 11, device)
    lw = _randn((T, k), g, device).double()
    out["topk_weights"] = torch.softmax(lw, dim=1).float()
    g = _gen(base + 12, "cpu")
    ids = torch.rand((T, 256), generator=g).argsort(dim=1)[:, :k].to(torch.int32)
    out["topk_ids"] = ids.to(device)
    if spec.shared:
        g = _gen(base + 5, device)
        out["shared"] = _randn((T, H), g, device).to(torch.bfloat16)
    if spec.residual:
        g = _gen(base + 7, device)
        out["residual"] = _randn((T, H), g, device).to(torch.bfloat16)
    if spec.rmsnorm:
        g = _gen(base + 8, device)
        out["gamma"] = (0.5 + torch.rand((H,), generator=g, device=device)).to(torch.bfloat16)
    return out


def to_numpy_bits(t):
    """Host numpy view of a stored tensor: bf16 -> uint16 bit patterns,
    fp8 codes stay uint8, float32/int32 unchanged."""
    if t is None:
        return None
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.contiguous().view(torch.uint8).numpy()
    return t.contiguous().numpy()
