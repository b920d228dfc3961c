"""The fused-MoE layer, step by step, as plain definitions (test
infrastructure only; see the package docstring).

Notation: T tokens, H hidden, I expert intermediate, E routed experts,
k = top_k, BM = align block size, flat index i = t*k + j for token t and slot
j.  bf16 tensors travel as uint16 bit patterns, fp8 tensors as uint8 OCP
E4M3 codes, everything else as numpy float32/int32.

Readings the pages leave open are stated where they are taken (the readings
table of the design notes lists them all):
  * routing is not on the pages: top-k by logit, ties to the lower expert
    index; softmax over all experts (optionally renormalised over the top-k)
    or sigmoid renormalised over the top-k;
  * the fp8 quantiser: per (token, 128-channel group) scale = amax/448 in
    float32 (amax floored at 1e-10), code = E4M3 round-to-nearest-even with
    saturation of value/scale computed in float32;
  * expert weights: W13 [E, 2I, H] with rows [0, I) = gate (W1) and rows
    [I, 2I) = up (W3); W2 [E, H, I]; fp8 weights carry one float32 scale per
    128x128 block of each matrix;
  * SiLU-mul: z = silu(gate) * up with silu(v) = v / (1 + exp(-v));
    silu_no_mul: z = silu(W1 a) with W13 holding only the I gate rows;
  * gelu / gelu_no_mul (the activation column of the fused-experts kernel
    table, which lists gelu_tanh separately): the exact GELU
    gelu(v) = v * Phi(v) = v/2 * (1 + erf(v / sqrt 2)), gated and ungated
    like silu;
  * the shared expert runs the same MLP on every token's unweighted input
    and is added with weight 1 in finalize.
"""

import numpy as np

from .codecs import (
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    e4m3_decode,
    e4m3_encode_sat,
    E4M3_MAX,
)

GROUP = 128          # G(128): per-token-group size for activations
WBLOCK = 128         # 128x128 weight-scale blocks
QUANT_EPS = np.float32(1e-10)


# --------------------------------------------------------------------------
# route
# --------------------------------------------------------------------------
def route(logits, top_k, scoring="softmax", renormalize=True):
    """Top-k routing.

    The pages only consume ``topk_ids``/``topk_weights`` (the no-DP/EP
    prepare and finalize signatures on "[vLLM] MoE Oracle & Prepare/
    Finalize"); the rule is the plain reading: per token, experts ordered by
    descending logit with ties to the lower expert index, the first k kept.
    Softmax and sigmoid are strictly increasing, so choosing on the float32
    logits is choosing on the scores, and the ids do not depend on how exp is
    rounded.

    Weights (float64, rounded once to float32):
      softmax, renormalised:  p_e = softmax(l)_e, w_j = p_{id_j} / sum_j' p_{id_j'}
      softmax, not renorm.:   w_j = softmax(l)_{id_j}
      sigmoid, renormalised:  w_j = sig(l_{id_j}) / sum_j' sig(l_{id_j'})
      sigmoid, not renorm.:   w_j = sig(l_{id_j})
    """
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    ld = l32.astype(np.float64)
    # A stable sort of -logit puts equal logits in ascending expert order.
    order = np.argsort(-ld, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)
    if scoring == "softmax":
        m = ld.max(axis=1, keepdims=True) if E else ld
        ex = np.exp(ld - m)
        p = ex / ex.sum(axis=1, keepdims=True)
    elif scoring == "sigmoid":
        p = 1.0 / (1.0 + np.exp(-ld))
    else:
        raise ValueError(scoring)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w.astype(np.float32)


# --------------------------------------------------------------------------
# prepare
# --------------------------------------------------------------------------
def quantize_g128(values):
    """fp8 E4M3 quantisation with one float32 scale per (row, 128-column
    group), the "G(128)" format of the pages' quant-format key.

    ``values`` (float64) are first taken to float32, the precision the
    kernels hold them in; the scale and the code are then decided in float32:
        amax = max |v| over the group,  s = max(amax, 1e-10) / 448,
        q = E4M3_rne_sat(v / s).
    Returns (codes uint8 [R, C], scales float32 [R, C/128])."""
    v32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    if C % GROUP:
        raise ValueError("columns must be a multiple of 128")
    g = v32.reshape(R, C // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if R else np.zeros((0, C // GROUP), np.float32)
    s = (np.maximum(amax, QUANT_EPS) / np.float32(E4M3_MAX)).astype(np.float32)
    scaled = (g / s[:, :, None]).astype(np.float32)
    q = e4m3_encode_sat(scaled.astype(np.float64))
    return q.reshape(R, C), s


def dequant_g128(codes, scales):
    """E4M3 codes [R, C] with G(128) scales [R, C/128] -> float64."""
    v = e4m3_decode(codes)
    return v * np.repeat(np.asarray(scales, np.float64), GROUP, axis=1)


def _quantize_scale(v32, amax):
    """E4M3 codes of float32 values v32 under float32 amax (broadcastable),
    with the scale rule of quantize_g128."""
    s = (np.maximum(amax, QUANT_EPS) / np.float32(E4M3_MAX)).astype(np.float32)
    q = e4m3_encode_sat((v32 / s).astype(np.float32).astype(np.float64))
    return q, s


def quantize_token(values):
    """fp8 E4M3 with one float32 scale per row over all its columns: the
    "A" (per activation token) format of the quant-format key.  Same scale
    and code rule as quantize_g128.  Returns (codes [R, C], scales [R, 1])."""
    v32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    amax = np.abs(v32).max(axis=1, keepdims=True) if v32.size else np.zeros((v32.shape[0], 1),
                                                                             np.float32)
    return _quantize_scale(v32, amax)


def quantize_tensor(values):
    """fp8 E4M3 with one float32 scale for the whole tensor: the "T" (per
    tensor) format of the quant-format key.  Returns (codes, scales [1, 1])."""
    v32 = np.asarray(values, dtype=np.float64).astype(np.float32)
    amax = np.abs(v32).max(keepdims=True).reshape(1, 1) if v32.size else np.zeros((1, 1),
                                                                                  np.float32)
    return _quantize_scale(v32, amax)


def dequant_scaled(codes, scales):
    """E4M3 codes [R, C] with scales in any of the three formats: G(128)
    [R, C/128], per token [R, 1] or per tensor [1, 1] -> float64."""
    scales = np.asarray(scales, np.float64)
    v = e4m3_decode(codes)
    C = v.shape[1]
    if scales.shape[1] == 1:
        return v * scales                     # broadcast over columns (and rows)
    if scales.shape[1] * GROUP != C:
        raise ValueError("scales do not match the G(128) layout")
    return v * np.repeat(scales, GROUP, axis=1)


# activation formats of prepare's fp8 quantiser
QUANTISERS = {"fp8": quantize_g128, "fp8_token": quantize_token, "fp8_tensor": quantize_tensor}


def prepare(x_bits, topk_weights, apply_router_weight_on_input, quant="none"):
    """No-DP/EP prepare ("[vLLM] MoE Oracle & Prepare/Finalize", the
    MoEPrepareAndFinalizeNoDPEPModular.prepare code): when the router weight
    goes on the input, top_k must be 1 and a1 = a1 * w with w first cast to
    the activation dtype (bf16); then the input quantiser runs.  Per the
    backend table's text, prepare's output is the quantised type.

    The bf16 x bf16 product is exact in float64, so the result has a single
    rounding.  quant="none" returns bf16 bits and no scales; quant="fp8"
    returns (codes, G(128) scales), "fp8_token" (codes, per-token scales
    [rows, 1]) and "fp8_tensor" (codes, one scale [1, 1])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    a_bits = x_bits
    if apply_router_weight_on_input:
        w = np.asarray(topk_weights, dtype=np.float32)
        if w.ndim != 2 or w.shape[1] != 1:
            raise ValueError("router weight on the input needs top_k == 1")
        wq = bf16_bits_to_f64(f64_to_bf16_bits(w.astype(np.float64)))
        a_bits = f64_to_bf16_bits(bf16_bits_to_f64(x_bits) * wq)
    if quant == "none":
        return a_bits, None
    if quant in QUANTISERS:
        return QUANTISERS[quant](bf16_bits_to_f64(a_bits))
    raise ValueError(quant)


# --------------------------------------------------------------------------
# align
# --------------------------------------------------------------------------
def align_capacity(T, top_k, E, block_m):
    """Sizes of the align outputs: sorted ids hold every flat index plus at
    most BM-1 pad slots for each expert that has rows (at most min(E, T*k)
    of them); block ids hold one entry per BM slots."""
    n = T * top_k
    cap = n + min(E, n) * (block_m - 1)
    return cap, -(-cap // block_m)


def align(topk_ids, E, block_m):
    """Sort the flat rows by expert into block-padded groups.

    The pages say only that the experts receive the tokens grouped per
    expert; the plain reading taken here:
      cnt[e]  = #{i : ids[i] == e}
      off[0] = 0, off[e+1] = off[e] + ceil(cnt[e] / BM) * BM
      sorted[off[e] + r] = the r-th flat index i (ascending) with ids[i] == e
      every other slot    = T*k (the pad sentinel)
      block[b] = e for b in [off[e]/BM, off[e+1]/BM), -1 beyond off[E]/BM
      num_tokens_post_padded = off[E]
    Returns a dict of int32 arrays."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = flat.size
    if n and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    cap, nblk = align_capacity(T, k, E, block_m)
    cnt = np.bincount(flat, minlength=E).astype(np.int64)
    padded = -(-cnt // block_m) * block_m
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(padded)
    sorted_ids = np.full(cap, n, dtype=np.int64)
    block = np.full(nblk, -1, dtype=np.int64)
    for e in range(E):
        rows = np.nonzero(flat == e)[0]          # ascending flat index
        sorted_ids[off[e]:off[e] + rows.size] = rows
        block[off[e] // block_m:off[e + 1] // block_m] = e
    return {
        "expert_counts": cnt.astype(np.int32),
        "expert_offsets": off.astype(np.int32),
        "sorted_token_ids": sorted_ids.astype(np.int32),
        "block_expert_ids": block.astype(np.int32),
        "num_tokens_post_padded": np.array([off[E]], dtype=np.int32),
    }


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(v):
    return v / (1.0 + np.exp(-v))


def gelu(v):
    """Exact GELU, v * Phi(v), with the standard normal CDF Phi written
    through erf (scipy's double-precision erf as the library primitive)."""
    from scipy.special import erf
    v = np.asarray(v, np.float64)
    return 0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))


_ACTS = {"silu": silu, "gelu": gelu}


def dequant_weight(w, scale):
    """One expert matrix [N, K] -> float64.  bf16 bits when ``scale`` is
    None, else E4M3 codes times one float32 scale per 128x128 block."""
    if scale is None:
        return bf16_bits_to_f64(w)
    v = e4m3_decode(w)
    s = np.asarray(scale, dtype=np.float64)
    N, K = v.shape
    if N % WBLOCK == 0 and K % WBLOCK == 0:
        # each 128x128 block times its scale (a view of v by blocks)
        blocks = v.reshape(N // WBLOCK, WBLOCK, K // WBLOCK, WBLOCK)
        blocks *= s[:N // WBLOCK, None, :K // WBLOCK, None]
        return v
    return v * np.repeat(np.repeat(s, WBLOCK, axis=0), WBLOCK, axis=1)[:N, :K]


def _scale_rows(scale, tok):
    """The scales of rows ``tok``: a single-row scale array (per tensor)
    serves every row."""
    if scale is None:
        return None
    scale = np.asarray(scale)
    return scale if scale.shape[0] == 1 else scale[tok]


def dequant_act(a, a_scale):
    """prepare's output -> float64 rows (any of the three fp8 scale formats)."""
    if a_scale is None:
        return bf16_bits_to_f64(a)
    return dequant_scaled(a, a_scale)


def _round_intermediate(z, mode, quant):
    """Where the kernels store the intermediate z (the pages are silent on
    its precision): "exact" keeps float64; "mirrored" rounds it to bf16 on
    the bf16 path, or to fp8 G(128) along I on the fp8 path (an fp8 second
    GEMM needs fp8 operands)."""
    if mode == "exact":
        return z
    if mode != "mirrored":
        raise ValueError(mode)
    if quant == "fp8":
        return dequant_g128(*quantize_g128(z))
    return bf16_bits_to_f64(f64_to_bf16_bits(z))


def expert_gemm1(a, w13, activation="silu"):
    """First half of one expert on rows ``a`` [n, H] (float64) with the
    dequantised W13 [2I or I, H]: h = a W13^T (library matmul, float64),
    then the activation.  Returns z [n, I] (float64, unrounded)."""
    h = a @ w13.T
    if callable(activation):        # a test-only activation without a gate/up split
        return activation(h)
    if activation in ("silu", "gelu"):
        inter = w13.shape[0] // 2
        return _ACTS[activation](h[:, :inter]) * h[:, inter:]
    if activation in ("silu_no_mul", "gelu_no_mul"):
        return _ACTS[activation[:-len("_no_mul")]](h)
    raise ValueError(activation)


def expert_gemm2(z, w2):
    """Second half: y = z W2^T with the dequantised W2 [H, I] (float64)."""
    return z @ w2.T


def expert_mlp(a, w13, w2, activation="silu", mode="exact", quant="none"):
    """One expert: y = W2 act(W13 a), with z rounded where the kernels store
    it when mode == "mirrored"."""
    z = expert_gemm1(a, w13, activation)
    z = _round_intermediate(z, mode, quant)
    return expert_gemm2(z, w2)


def experts(a1q, a1q_scale, topk_ids, w13, w13_scale, w2, w2_scale,
            activation="silu", mode="exact", shared=None, tokens=None):
    """The experts stage: for every flat row i = t*k + j with e = ids[t, j],
    y = W2[e] act(W13[e] a[t]); the output keeps the original activation
    dtype (bf16) in the [T, k, H] slot layout.

    ``shared`` (optional) = dict(a=..., a_scale=..., w13=..., w13_scale=...,
    w2=..., w2_scale=...): the always-on shared expert, run on every token's
    (unweighted) input, returned as bf16 [T, H].

    ``tokens`` (optional) restricts the work to a subset of token indices:
    each token's rows depend on nothing but that token, so a subset is a
    valid sample of the full result.  Rows of tokens outside the subset are
    left at zero.  Returns (fused_expert_output bits [T, k, H],
    shared_out bits [T, H] or None)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    quant = "none" if a1q_scale is None else "fp8"
    H = a1q.shape[1]
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.zeros((T, k, H), dtype=np.uint16)
    a_tok = dequant_act(a1q[tok], _scale_rows(a1q_scale, tok))
    sub_ids = ids[tok]                                   # [n, k]
    for e in np.unique(sub_ids):
        rr, jj = np.nonzero(sub_ids == e)                # rows of the subset
        w13e = dequant_weight(w13[e], None if w13_scale is None else w13_scale[e])
        w2e = dequant_weight(w2[e], None if w2_scale is None else w2_scale[e])
        y = expert_mlp(a_tok[rr], w13e, w2e, activation, mode, quant)
        out[tok[rr], jj] = f64_to_bf16_bits(y)
    shared_out = None
    if shared is not None:
        sa = shared["a"][tok]
        ss = shared.get("a_scale")
        a_sh = dequant_act(sa, _scale_rows(ss, tok))
        w13s = dequant_weight(shared["w13"], shared.get("w13_scale"))
        w2s = dequant_weight(shared["w2"], shared.get("w2_scale"))
        y = expert_mlp(a_sh, w13s, w2s, activation, mode, quant)
        shared_out = np.zeros((T, H), dtype=np.uint16)
        shared_out[tok] = f64_to_bf16_bits(y)
    return out, shared_out


def experts_batched(a, a_scale, expert_num_tokens, w13, w13_scale, w2, w2_scale,
                    activation="silu", mode="exact", experts_subset=None):
    """The experts stage on the batched activation format: prepare may hand
    the experts one batch per expert instead of the token-major rows ("Fused
    MoE Kernel Features": the standard and batched output formats of
    prepare, and the batched experts kernels of the fused-experts table).
    Batch e holds expert e's input rows in its first count[e] positions;
    for each of them y = W2[e] act(W13[e] a[e, m]) in bf16, the same MLP the
    standard-format stage runs per routed row.  Positions past the count
    carry nothing and stay zero here.  Reading: a count outside [0, M] is
    clamped into it (a batch has M rows).

    a [E, M, H] bf16 bits or E4M3 codes; a_scale None (bf16) or the fp8
    scales as [E, M, H/128] (G(128)), [E, M, 1] (per token) or [1, 1] (per
    tensor).  ``experts_subset`` restricts the work to some experts (the
    others' batches stay zero).  Returns out bits [E, M, H]."""
    a = np.asarray(a)
    E, M, H = a.shape
    counts = np.clip(np.asarray(expert_num_tokens, dtype=np.int64), 0, M)
    quant = "none" if a_scale is None else "fp8"
    out = np.zeros((E, M, H), dtype=np.uint16)
    for e in (range(E) if experts_subset is None else experts_subset):
        c = int(counts[e])
        if c == 0:
            continue
        s = None
        if a_scale is not None:
            s = np.asarray(a_scale)
            s = s if s.ndim == 2 else s[e, :c]
        rows = dequant_act(a[e, :c], s)
        w13e = dequant_weight(w13[e], None if w13_scale is None else w13_scale[e])
        w2e = dequant_weight(w2[e], None if w2_scale is None else w2_scale[e])
        out[e, :c] = f64_to_bf16_bits(expert_mlp(rows, w13e, w2e, activation, mode, quant))
    return out


# --------------------------------------------------------------------------
# finalize
# --------------------------------------------------------------------------
def finalize(fused_expert_output, topk_weights, apply_router_weight_on_input,
             shared=None, residual=None, gamma=None, eps=1e-6, out_quant="none",
             tokens=None):
    """No-DP/EP finalize: the weight-and-reduce step over the top-k expert
    rows ("[vLLM] MoE Oracle & Prepare/Finalize"), with the fusions of the
    flashinfer finalize program ("[flashinfer] MoE Finalize + AllReduce ..."
    introduction): optional shared-expert row, residual add and RMSNorm.

      acc[t] = sum_j w'[t, j] * y[t, j]   (slot order; w' = 1 when the
               weight was already applied on the input -- the pages apply it
               to the input *instead of* the output)
             + shared[t] + residual[t]    (each optional, weight 1)
      out[t] = acc[t] / sqrt(mean_d acc[t]^2 + eps) * gamma   if gamma given,
               acc[t] otherwise
    out is bf16, or fp8 E4M3 with G(128) scales (the quantiser of
    ``quantize_g128``).  residual_out = bf16(acc).  Float64 throughout.
    Returns (out_bits_or_codes, out_scales_or_None, residual_out_bits)."""
    y = bf16_bits_to_f64(fused_expert_output)          # [T, k, H]
    T, k, H = y.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = y[tok]
    if apply_router_weight_on_input:
        w = np.ones((tok.size, k))
    else:
        w = np.asarray(topk_weights, dtype=np.float32)[tok].astype(np.float64)
    acc = np.zeros((tok.size, H))
    for j in range(k):
        acc += w[:, j:j + 1] * y[:, j, :]
    if shared is not None:
        acc += bf16_bits_to_f64(shared)[tok]
    if residual is not None:
        acc += bf16_bits_to_f64(residual)[tok]
    if gamma is not None:
        r = 1.0 / np.sqrt((acc * acc).mean(axis=1, keepdims=True) + eps)
        out = acc * r * bf16_bits_to_f64(gamma)[None, :]
    else:
        out = acc
    res_out = f64_to_bf16_bits(acc)
    if out_quant == "none":
        return f64_to_bf16_bits(out), None, res_out
    if out_quant == "fp8":
        q, s = quantize_g128(out)
        return q, s, res_out
    raise ValueError(out_quant)


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def forward(x_bits, logits, w, top_k, scoring, renormalize, block_m,
            apply_router_weight_on_input=False, quant="none", activation="silu",
            mode="mirrored", residual=None, gamma=None, eps=1e-6,
            out_quant="none", tokens=None):
    """route -> prepare -> align -> experts -> finalize.

    ``w``: dict with w13, w2 (and w13_scale, w2_scale on the fp8 path) and
    optionally shared_w13, shared_w2 (+ scales).  The shared expert takes the
    unweighted input, quantised like a1q.  Returns a dict of every stage's
    outputs; with ``tokens`` given, routing and align cover all tokens and
    the rest covers the subset only."""
    ids, tw = route(logits, top_k, scoring, renormalize)
    E = w["w13"].shape[0]
    al = align(ids, E, block_m)
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    tok = np.arange(x_bits.shape[0]) if tokens is None else np.asarray(tokens)
    T, H = x_bits.shape

    def prep(weights):
        # the per-tensor scale depends on every token: quantise them all
        if quant == "fp8_tensor":
            return prepare(x_bits, weights, apply_router_weight_on_input and weights is not None,
                           quant)
        a_sub, s_sub = prepare(x_bits[tok], None if weights is None else weights[tok],
                               apply_router_weight_on_input and weights is not None, quant)
        a = np.zeros((T, H), dtype=a_sub.dtype)
        a[tok] = a_sub
        if s_sub is None:
            return a, None
        sc = np.zeros((T, s_sub.shape[1]), dtype=np.float32)
        sc[tok] = s_sub
        return a, sc

    a1q, a1q_scale = prep(tw)
    shared = None
    if w.get("shared_w13") is not None:
        if apply_router_weight_on_input:
            sa, ss = prep(None)
        else:
            sa, ss = a1q, a1q_scale
        shared = dict(a=sa, a_scale=ss, w13=w["shared_w13"], w13_scale=w.get("shared_w13_scale"),
                      w2=w["shared_w2"], w2_scale=w.get("shared_w2_scale"))
    feo, sh_out = experts(a1q, a1q_scale, ids, w["w13"], w.get("w13_scale"), w["w2"],
                          w.get("w2_scale"), activation, mode, shared, tokens=tok)
    out, out_s, res_out = finalize(feo, tw, apply_router_weight_on_input, sh_out,
                                   residual, gamma, eps, out_quant, tokens=tok)
    return dict(topk_ids=ids, topk_weights=tw, align=al, a1q=a1q, a1q_scale=a1q_scale,
                fused_expert_output=feo, shared_out=sh_out, output=out,
                output_scale=out_s, residual_out=res_out, tokens=tok)
