"""Thin ctypes binding of libmoe.so: the C entry points under the same names.

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the layer runs in the library's kernels.
Outputs that the caller does not pass are allocated here with torch (device
memory is torch's job), workspaces likewise.  A missing library raises at
import time -- there is no fallback path.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4

SCORING = {"softmax": 0, "sigmoid": 1}
QUANT = {"none": 0, "fp8": 1, "fp8_token": 2, "fp8_tensor": 3}


def _is_fp8(quant):
    return quant in ("fp8", "fp8_token", "fp8_tensor")


def _act_scale_shape(quant, T, H):
    """fp32 scales of an fp8 [T, H] activation: G(128), per token, per tensor."""
    return {"fp8": (T, H // 128), "fp8_token": (T,), "fp8_tensor": (1,)}[quant]
ACTIVATION = {"silu": 0, "silu_no_mul": 1, "gelu": 2, "gelu_no_mul": 3}
NUM_STAGE_EVENTS = 8
STAGES = ("start", "route", "prepare", "align", "gemm1", "gemm2", "shared", "finalize")

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_int = ctypes.c_int


class MoeWeights(ctypes.Structure):
    _fields_ = [("num_experts", c_i32), ("inter", c_i32), ("quant", c_i32), ("shared_inter", c_i32),
                ("w13", c_vp), ("w13_scale", c_vp), ("w2", c_vp), ("w2_scale", c_vp),
                ("shared_w13", c_vp), ("shared_w13_scale", c_vp), ("shared_w2", c_vp),
                ("shared_w2_scale", c_vp)]


class MoeQuantConfig(ctypes.Structure):
    _fields_ = [("quant", c_i32), ("act_group", c_i32), ("w_block_n", c_i32), ("w_block_k", c_i32)]


def quant_config(quant="none", act_group=None, w_block_n=128, w_block_k=128):
    """The prepare quant_config: the format, its activation group (128 for
    G(128), 0 for per token / per tensor) and the 128x128 weight blocks."""
    if act_group is None:
        act_group = 128 if quant == "fp8" else 0
    return MoeQuantConfig(QUANT[quant], act_group, w_block_n, w_block_k)


class MoeError(RuntimeError):
    def __init__(self, status, fn, msg):
        super().__init__(f"{fn} -> {status_str(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python mixture_experts_layer_routing_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "moe_status_str": (ctypes.c_char_p, [c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_pick_block_m": (c_int, [c_int, c_int, c_int, c_int]),
        "moe_route": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp]),
        "moe_prepare": (c_int, [c_vp, c_int, c_int, c_vp, c_vp, c_int, c_int,
                                ctypes.POINTER(MoeQuantConfig), c_vp, c_vp, c_vp]),
        "moe_align": (c_int, [c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                              c_vp, c_sz, c_vp]),
        "moe_align_capacity": (c_int, [c_int, c_int, c_int, c_int, ctypes.POINTER(c_i64),
                                       ctypes.POINTER(c_i64)]),
        "moe_align_workspace_bytes": (c_sz, [c_int, c_int, c_int, c_int]),
        "moe_experts": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                ctypes.POINTER(MoeWeights), c_int, c_vp, c_vp, c_vp, c_int,
                                c_vp, c_vp, c_vp, c_sz, c_vp]),
        "moe_experts_workspace_bytes": (c_sz, [c_int, c_int, c_int, ctypes.POINTER(MoeWeights),
                                               c_int, c_int]),
        "moe_experts_workspace_layout": (c_int, [c_int, c_int, c_int, ctypes.POINTER(MoeWeights),
                                                 c_int, c_int, ctypes.POINTER(c_sz)]),
        "moe_experts_batched": (c_int, [c_vp, c_vp, c_vp, c_int, c_int, ctypes.POINTER(MoeWeights),
                                        c_int, c_int, c_vp, c_vp, c_sz, c_vp]),
        "moe_experts_batched_workspace_bytes": (c_sz, [c_int, c_int, ctypes.POINTER(MoeWeights),
                                                       c_int, c_int]),
        "moe_experts_batched_workspace_layout": (c_int, [c_int, c_int, ctypes.POINTER(MoeWeights),
                                                         c_int, c_int, ctypes.POINTER(c_sz)]),
        "moe_finalize": (c_int, [c_vp, c_vp, c_int, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                 c_vp, c_vp, c_vp, c_vp, c_f32, c_vp]),
        "moe_forward": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                ctypes.POINTER(MoeWeights), c_int, c_int, c_vp, c_vp, c_f32, c_int,
                                c_vp, c_vp, c_vp, c_vp, c_sz, c_vp, c_vp]),
        "moe_forward_workspace_bytes": (c_sz, [c_int, c_int, c_int, ctypes.POINTER(MoeWeights),
                                               c_int, c_int, c_int]),
        "moe_forward_noalloc": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                        ctypes.POINTER(MoeWeights), c_int, c_int, c_vp, c_vp, c_f32,
                                        c_int, c_vp, c_vp, c_vp, c_vp]),
        "moe_forward_graph_create": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                             ctypes.POINTER(MoeWeights), c_int, c_int, c_vp, c_vp,
                                             c_f32, c_int, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp,
                                             ctypes.POINTER(c_vp)]),
        "moe_forward_monolithic": (c_int, [c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                           ctypes.POINTER(MoeWeights), c_int, c_vp, c_vp, c_f32,
                                           c_int, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
        "moe_forward_monolithic_workspace_bytes": (c_sz, [c_int, c_int, c_int,
                                                          ctypes.POINTER(MoeWeights), c_int]),
        "moe_forward_graph_launch": (c_int, [c_vp, c_vp]),
        "moe_forward_graph_destroy": (c_int, [c_vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def status_str(status):
    return _lib.moe_status_str(status).decode()


def last_error():
    return _lib.moe_last_error().decode()


def _check(status, fn):
    if status != MOE_OK:
        raise MoeError(status, fn, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _quant_of(t):
    return 1 if t.dtype in (torch.uint8, torch.float8_e4m3fn) else 0


def make_weights(w13, w2, w13_scale=None, w2_scale=None, shared_w13=None, shared_w2=None,
                 shared_w13_scale=None, shared_w2_scale=None, quant=None):
    """Host struct of device pointers; the tensors must stay alive while it is used.
    ``quant`` names the activation format for fp8 weights ("fp8" = G(128),
    "fp8_token", "fp8_tensor"); by default it follows the weight dtype."""
    w = MoeWeights()
    w.num_experts = w13.shape[0]
    w.inter = w2.shape[2]
    w.quant = _quant_of(w13) if quant is None else QUANT[quant]
    w.shared_inter = 0 if shared_w2 is None else shared_w2.shape[1]
    w.w13, w.w13_scale, w.w2, w.w2_scale = _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale)
    w.shared_w13, w.shared_w13_scale = _ptr(shared_w13), _ptr(shared_w13_scale)
    w.shared_w2, w.shared_w2_scale = _ptr(shared_w2), _ptr(shared_w2_scale)
    w._keep = (w13, w2, w13_scale, w2_scale, shared_w13, shared_w2, shared_w13_scale, shared_w2_scale)
    return w


def moe_pick_block_m(T, top_k, num_experts, quant="none"):
    return _lib.moe_pick_block_m(T, top_k, num_experts, QUANT[quant])


def moe_align_capacity(T, top_k, E, block_m):
    s, b = c_i64(), c_i64()
    _check(_lib.moe_align_capacity(T, top_k, E, block_m, ctypes.byref(s), ctypes.byref(b)),
           "moe_align_capacity")
    return s.value, b.value


def moe_route(logits, top_k, scoring="softmax", renormalize=True, topk_ids=None,
              topk_weights=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check(_lib.moe_route(_ptr(logits), T, E, top_k, SCORING[scoring], int(renormalize),
                          _ptr(topk_ids), _ptr(topk_weights), _stream(stream)), "moe_route")
    return topk_ids, topk_weights


def moe_prepare(a1, topk_weights=None, topk_ids=None, apply_router_weight_on_input=False,
                quant="none", a1q=None, a1q_scale=None, stream=None, qc=None):
    """prepare(a1, topk_weights, topk_ids, apply_router_weight_on_input,
    quant_config) -> (a1q, a1q_scale or None).  ``qc`` (a MoeQuantConfig)
    overrides the config built from ``quant``; ``topk_ids`` is passed through
    to the library, which does not read it without expert parallelism."""
    T, H = a1.shape
    dev = a1.device
    qc = quant_config(quant) if qc is None else qc
    quant = {v: k for k, v in QUANT.items()}.get(qc.quant, quant)
    top_k = (topk_weights.shape[1] if topk_weights is not None
             else (topk_ids.shape[1] if topk_ids is not None else 1))
    if a1q is None:
        a1q = torch.empty((T, H), dtype=torch.uint8 if _is_fp8(quant) else torch.bfloat16,
                          device=dev)
    if _is_fp8(quant) and a1q_scale is None:
        a1q_scale = torch.empty(_act_scale_shape(quant, T, H), dtype=torch.float32, device=dev)
    _check(_lib.moe_prepare(_ptr(a1), T, H, _ptr(topk_weights), _ptr(topk_ids), top_k,
                            int(apply_router_weight_on_input), ctypes.byref(qc), _ptr(a1q),
                            _ptr(a1q_scale), _stream(stream)), "moe_prepare")
    return a1q, (a1q_scale if _is_fp8(quant) else None)


def moe_align(topk_ids, E, block_m, stream=None, out=None, workspace=None):
    """Returns a dict of the align outputs; ``out`` (such a dict from an
    earlier call of the same shape) and ``workspace`` are reused when given."""
    T, k = topk_ids.shape
    dev = topk_ids.device
    if out is None:
        scap, bcap = moe_align_capacity(T, k, E, block_m)
        out = {
            "expert_counts": torch.empty(E, dtype=torch.int32, device=dev),
            "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "sorted_token_ids": torch.empty(scap, dtype=torch.int32, device=dev),
            "block_expert_ids": torch.empty(bcap, dtype=torch.int32, device=dev),
            "num_tokens_post_padded": torch.empty(1, dtype=torch.int32, device=dev),
        }
    wsb = _lib.moe_align_workspace_bytes(T, k, E, block_m)
    ws = workspace if workspace is not None else out.get("_ws")
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(_lib.moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(out["expert_counts"]),
                          _ptr(out["expert_offsets"]), _ptr(out["sorted_token_ids"]),
                          _ptr(out["block_expert_ids"]), _ptr(out["num_tokens_post_padded"]),
                          _ptr(ws), wsb, _stream(stream)), "moe_align")
    out["_ws"] = ws
    return out


def moe_experts(a1q, a1q_scale, weights, top_k, align_out, block_m, activation="silu",
                shared_in=None, shared_in_scale=None, fused_expert_output=None, shared_out=None,
                workspace=None, stream=None):
    """Returns (fused_expert_output, shared_out); with ``workspace`` given
    (a uint8 tensor) the intermediate z stays readable in it afterwards
    (see moe_experts_workspace_layout)."""
    T, H = a1q.shape
    dev = a1q.device
    if fused_expert_output is None:
        fused_expert_output = torch.empty((T, top_k, H), dtype=torch.bfloat16, device=dev)
    if weights.shared_inter > 0 and shared_out is None:
        shared_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    act = ACTIVATION[activation]
    wsb = _lib.moe_experts_workspace_bytes(T, H, top_k, ctypes.byref(weights), act, block_m)
    ws = workspace
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    if weights.shared_inter > 0 and shared_in is None:
        shared_in, shared_in_scale = a1q, a1q_scale
    _check(_lib.moe_experts(_ptr(a1q), _ptr(a1q_scale), _ptr(shared_in), _ptr(shared_in_scale), T, H,
                            top_k, ctypes.byref(weights), act, _ptr(align_out["sorted_token_ids"]),
                            _ptr(align_out["block_expert_ids"]),
                            _ptr(align_out["num_tokens_post_padded"]), block_m,
                            _ptr(fused_expert_output), _ptr(shared_out), _ptr(ws), wsb,
                            _stream(stream)), "moe_experts")
    return fused_expert_output, shared_out


def moe_experts_workspace_layout(T, H, top_k, weights, activation="silu", block_m=16):
    """Byte offsets of the intermediate z (and scales) inside moe_experts'
    workspace: dict(z, z_scale, shared_z, shared_z_scale, rows); None = absent."""
    out = (c_sz * 5)()
    _check(_lib.moe_experts_workspace_layout(T, H, top_k, ctypes.byref(weights),
                                             ACTIVATION[activation], block_m, out),
           "moe_experts_workspace_layout")
    none = (1 << (8 * ctypes.sizeof(c_sz))) - 1
    v = [None if x == none else x for x in out]
    return dict(z=v[0], z_scale=v[1], shared_z=v[2], shared_z_scale=v[3], rows=v[4])


def moe_experts_batched(a, a_scale, expert_num_tokens, weights, activation="silu", block_m=0,
                        out=None, workspace=None, stream=None):
    """Experts on the batched format: ``a`` [E, M, H] (bf16, or E4M3 codes
    as uint8 with ``a_scale`` in weights' format), ``expert_num_tokens`` [E]
    int32.  Returns ``out`` [E, M, H] bf16; rows past an expert's count are
    left as they were (uninitialised when ``out`` is not given).  With
    ``workspace`` given (a uint8 tensor) the schedule and z stay readable in
    it afterwards (see moe_experts_batched_workspace_layout)."""
    E, M, H = a.shape
    dev = a.device
    if out is None:
        out = torch.empty((E, M, H), dtype=torch.bfloat16, device=dev)
    act = ACTIVATION[activation]
    wsb = _lib.moe_experts_batched_workspace_bytes(M, H, ctypes.byref(weights), act, block_m)
    ws = workspace
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(_lib.moe_experts_batched(_ptr(a), _ptr(a_scale), _ptr(expert_num_tokens), M, H,
                                    ctypes.byref(weights), act, block_m, _ptr(out), _ptr(ws), wsb,
                                    _stream(stream)), "moe_experts_batched")
    return out


def moe_experts_batched_workspace_layout(M, H, weights, activation="silu", block_m=0):
    """Byte offsets inside moe_experts_batched's workspace: dict(sorted, z,
    z_scale, rows); None = absent."""
    out = (c_sz * 4)()
    _check(_lib.moe_experts_batched_workspace_layout(M, H, ctypes.byref(weights),
                                                     ACTIVATION[activation], block_m, out),
           "moe_experts_batched_workspace_layout")
    none = (1 << (8 * ctypes.sizeof(c_sz))) - 1
    v = [None if x == none else x for x in out]
    return dict(sorted=v[0], z=v[1], z_scale=v[2], rows=v[3])


def moe_finalize(fused_expert_output, topk_weights, topk_ids=None,
                 apply_router_weight_on_input=False, shared=None, residual=None, gamma=None,
                 eps=1e-6, out_quant="none", output=None, output_scale=None, residual_out=None,
                 want_residual_out=False, stream=None):
    T, k, H = fused_expert_output.shape
    dev = fused_expert_output.device
    if output is None:
        output = torch.empty((T, H), dtype=torch.uint8 if out_quant == "fp8" else torch.bfloat16,
                             device=dev)
    if out_quant == "fp8" and output_scale is None:
        output_scale = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    if want_residual_out and residual_out is None:
        residual_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(_lib.moe_finalize(_ptr(output), _ptr(output_scale), QUANT[out_quant],
                             _ptr(fused_expert_output), _ptr(topk_weights), _ptr(topk_ids), T, k, H,
                             int(apply_router_weight_on_input), _ptr(shared), _ptr(residual),
                             _ptr(residual_out), _ptr(gamma), float(eps), _stream(stream)),
           "moe_finalize")
    return output, (output_scale if out_quant == "fp8" else None), residual_out


def moe_forward_workspace_bytes(T, H, top_k, weights, activation="silu", block_m=0,
                                apply_router_weight_on_input=False):
    return _lib.moe_forward_workspace_bytes(T, H, top_k, ctypes.byref(weights),
                                            ACTIVATION[activation], block_m,
                                            int(apply_router_weight_on_input))


def moe_forward(x, logits, weights, top_k, scoring="softmax", renormalize=True,
                apply_router_weight_on_input=False, activation="silu", block_m=0, residual=None,
                gamma=None, eps=1e-6, out_quant="none", output=None, output_scale=None,
                residual_out=None, workspace=None, stage_events=None, stream=None):
    T, H = x.shape
    dev = x.device
    if output is None:
        output = torch.empty((T, H), dtype=torch.uint8 if out_quant == "fp8" else torch.bfloat16,
                             device=dev)
    if out_quant == "fp8" and output_scale is None:
        output_scale = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    wsb = moe_forward_workspace_bytes(T, H, top_k, weights, activation, block_m,
                                      apply_router_weight_on_input)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {NUM_STAGE_EVENTS} events")
        for e in stage_events:
            if e.cuda_event == 0:      # torch creates the HIP event on its first record
                e.record(stream if stream is not None else torch.cuda.current_stream())
        ev = (c_vp * NUM_STAGE_EVENTS)(*[e.cuda_event for e in stage_events])
    _check(_lib.moe_forward(_ptr(x), _ptr(logits), T, H, top_k, SCORING[scoring], int(renormalize),
                            int(apply_router_weight_on_input), ctypes.byref(weights),
                            ACTIVATION[activation], block_m, _ptr(residual), _ptr(gamma),
                            float(eps), QUANT[out_quant], _ptr(output), _ptr(output_scale),
                            _ptr(residual_out), _ptr(workspace), wsb, ev, _stream(stream)),
           "moe_forward")
    return output, (output_scale if out_quant == "fp8" else None), workspace


def moe_forward_monolithic(x, logits, weights, top_k, scoring="softmax", renormalize=True,
                           apply_router_weight_on_input=False, activation="silu", residual=None,
                           gamma=None, eps=1e-6, out_quant="none", output=None, output_scale=None,
                           residual_out=None, workspace=None, stream=None):
    """The whole layer as one kernel launch (bf16 weights, T <= 512,
    T*top_k <= 512); arguments and results as moe_forward."""
    T, H = x.shape
    dev = x.device
    if output is None:
        output = torch.empty((T, H), dtype=torch.uint8 if out_quant == "fp8" else torch.bfloat16,
                             device=dev)
    if out_quant == "fp8" and output_scale is None:
        output_scale = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    wsb = _lib.moe_forward_monolithic_workspace_bytes(T, H, top_k, ctypes.byref(weights),
                                                      ACTIVATION[activation])
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    _check(_lib.moe_forward_monolithic(
        _ptr(x), _ptr(logits), T, H, top_k, SCORING[scoring], int(renormalize),
        int(apply_router_weight_on_input), ctypes.byref(weights), ACTIVATION[activation],
        _ptr(residual), _ptr(gamma), float(eps), QUANT[out_quant], _ptr(output),
        _ptr(output_scale), _ptr(residual_out), _ptr(workspace), wsb, _stream(stream)),
        "moe_forward_monolithic")
    return output, (output_scale if out_quant == "fp8" else None), workspace


NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(x, logits, weights, top_k, scoring="softmax", renormalize=True,
                        apply_router_weight_on_input=False, activation="silu", block_m=0,
                        residual=None, gamma=None, eps=1e-6, out_quant="none", output=None,
                        output_scale=None, residual_out=None, stream=None):
    """moe_forward on the library's fixed per-GPU scratch: the library
    allocates nothing (outputs not passed in are allocated here by torch)."""
    T, H = x.shape
    dev = x.device
    if output is None:
        output = torch.empty((T, H), dtype=torch.uint8 if out_quant == "fp8" else torch.bfloat16,
                             device=dev)
    if out_quant == "fp8" and output_scale is None:
        output_scale = torch.empty((T, H // 128), dtype=torch.float32, device=dev)
    _check(_lib.moe_forward_noalloc(_ptr(x), _ptr(logits), T, H, top_k, SCORING[scoring],
                                    int(renormalize), int(apply_router_weight_on_input),
                                    ctypes.byref(weights), ACTIVATION[activation], block_m,
                                    _ptr(residual), _ptr(gamma), float(eps), QUANT[out_quant],
                                    _ptr(output), _ptr(output_scale), _ptr(residual_out),
                                    _stream(stream)), "moe_forward_noalloc")
    return output, (output_scale if out_quant == "fp8" else None)


class ForwardGraph:
    """moe_forward captured once into a HIP graph (moe_forward_graph_create)
    and replayed with one launch.  The graph is bound to the tensors given
    here: write new inputs into ``x`` / ``logits`` (and ``residual``,
    ``gamma``) in place, call launch(), then read ``output``.  Capture runs on
    ``stream`` (default: the current stream), which must not be the null
    stream."""

    def __init__(self, x, logits, weights, top_k, scoring="softmax", renormalize=True,
                 apply_router_weight_on_input=False, activation="silu", block_m=0, residual=None,
                 gamma=None, eps=1e-6, out_quant="none", want_residual_out=False, stream=None):
        T, H = x.shape
        dev = x.device
        self.output = torch.empty((T, H), dtype=torch.uint8 if out_quant == "fp8" else torch.bfloat16,
                                  device=dev)
        self.output_scale = (torch.empty((T, H // 128), dtype=torch.float32, device=dev)
                             if out_quant == "fp8" else None)
        self.residual_out = (torch.empty((T, H), dtype=torch.bfloat16, device=dev)
                             if want_residual_out else None)
        wsb = moe_forward_workspace_bytes(T, H, top_k, weights, activation, block_m,
                                          apply_router_weight_on_input)
        self.workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
        self._keep = (x, logits, weights, residual, gamma)
        self._h = c_vp()
        st = stream if stream is not None else torch.cuda.current_stream()
        if st.cuda_stream == 0:
            raise ValueError("graph capture needs a created stream, not the null stream")
        _check(_lib.moe_forward_graph_create(
            _ptr(x), _ptr(logits), T, H, top_k, SCORING[scoring], int(renormalize),
            int(apply_router_weight_on_input), ctypes.byref(weights), ACTIVATION[activation],
            block_m, _ptr(residual), _ptr(gamma), float(eps), QUANT[out_quant], _ptr(self.output),
            _ptr(self.output_scale), _ptr(self.residual_out), _ptr(self.workspace), wsb,
            _stream(st), ctypes.byref(self._h)), "moe_forward_graph_create")

    def launch(self, stream=None):
        """Enqueue one replay; returns (output, output_scale)."""
        if not self._h:
            raise RuntimeError("graph was closed")
        _check(_lib.moe_forward_graph_launch(self._h, _stream(stream)), "moe_forward_graph_launch")
        return self.output, self.output_scale

    def close(self):
        """Wait for pending replays, then release the graph."""
        if self._h:
            torch.cuda.synchronize(self.output.device)
            h, self._h = self._h, c_vp()
            _check(_lib.moe_forward_graph_destroy(h), "moe_forward_graph_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
