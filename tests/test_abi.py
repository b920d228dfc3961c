"""The C ABI on the host: libmoe.so loads, exports every function moe.h
declares, and its pure host paths (capacities, workspace sizes, block-size
choice, argument validation) behave as documented.  No kernel runs here."""

import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_routing_amd as m
    return m


def test_header_declares_the_six_stage_calls():
    names = _declared_functions()
    for f in ("moe_route", "moe_prepare", "moe_align", "moe_experts", "moe_finalize", "moe_forward"):
        assert f in names


def test_library_exports_every_declared_function(moe):
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(moe):
    assert moe.status_str(0) == "MOE_OK"
    assert moe.status_str(1) == "MOE_ERR_INVALID_ARG"
    assert moe.status_str(4) == "MOE_ERR_HIP"
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("T,k,E,BM", [(16, 2, 8, 16), (4096, 2, 8, 128), (1, 2, 8, 16),
                                      (8192, 8, 256, 64), (0, 2, 8, 16), (3, 1, 1024, 256)])
def test_align_capacity_matches_oracle(moe, T, k, E, BM):
    assert moe.moe_align_capacity(T, k, E, BM) == oracle.align_capacity(T, k, E, BM)


def test_pick_block_m(moe):
    assert moe.moe_pick_block_m(1, 2, 8) == 16
    assert moe.moe_pick_block_m(512, 2, 8) == 256
    assert moe.moe_pick_block_m(256, 2, 8) == 64
    assert moe.moe_pick_block_m(4096, 2, 8) == 256
    assert moe.moe_pick_block_m(4096, 2, 8, "fp8") == 256
    assert moe.moe_pick_block_m(640, 2, 8, "fp8") == 128
    assert moe.moe_pick_block_m(64, 8, 256, "fp8") == 16
    assert moe.moe_pick_block_m(8192, 8, 256, "fp8") == 256
    assert moe.moe_pick_block_m(4096, 8, 256, "fp8") == 128


def test_align_workspace_is_zero_for_one_tile(moe):
    lib = moe.binding.lib()
    assert lib.moe_align_workspace_bytes(16, 2, 8, 16) == 0
    assert lib.moe_align_workspace_bytes(4096, 8, 256, 16) == 0          # 32768 ids: one workgroup
    # 65536 ids: 32 tiles of 2048 (8 wave counts + 1 tile total per tile and expert)
    assert lib.moe_align_workspace_bytes(8192, 8, 256, 16) == (32 * 9 + 1) * 256 * 4
    # 2^24 ids: 2048 tiles of 8192 (the LDS-sized maximum)
    assert lib.moe_align_workspace_bytes(1 << 21, 8, 256, 128) == (2048 * 9 + 1) * 256 * 4
    assert lib.moe_align_workspace_bytes(1 << 23, 2, 8, 256) == (2048 * 9 + 1) * 8 * 4
    # 2^20 ids: 512 tiles of 2048; 2^22: 1024 of 4096
    assert lib.moe_align_workspace_bytes(1 << 17, 8, 64, 64) == (512 * 9 + 1) * 64 * 4
    assert lib.moe_align_workspace_bytes(1 << 21, 2, 8, 256) == (1024 * 9 + 1) * 8 * 4
    # 40000 ids, E=2: 20 tiles of 2048 need less than the one-launch path's
    # 257 64-bit flags and the expert counts of up to 10 tiles of 4096
    assert lib.moe_align_workspace_bytes(20000, 2, 2, 16) == 8 * 257 + 4 * 10 * 2


def _bad(moe, fn, *args):
    return getattr(moe.binding.lib(), fn)(*args)


def test_validation_happens_before_any_launch(moe):
    L = moe.binding.lib()
    null = None
    # top_k > E, E out of range, bad scoring
    assert L.moe_route(null, 4, 8, 9, 0, 1, null, null, null) == 1
    assert L.moe_route(null, 4, 0, 1, 0, 1, null, null, null) == 1
    assert L.moe_route(null, 4, 8, 2, 7, 1, null, null, null) == 1
    # T == 0 is a no-op and touches no pointer
    assert L.moe_route(null, 0, 8, 2, 0, 1, null, null, null) == 0
    # prepare(a1, topk_weights, topk_ids, ..., apply_router_weight_on_input,
    # quant_config): weight on the input needs top_k == 1 (the pages' assert)
    qc = moe.binding.quant_config
    none, g128 = ctypes.byref(qc("none")), ctypes.byref(qc("fp8"))
    assert L.moe_prepare(null, 4, 128, null, null, 2, 1, none, null, null, null) == 1
    assert "top_k == 1" in moe.last_error()
    # fp8 needs H % 128 == 0; an unknown quant is unsupported; no config at all
    assert L.moe_prepare(null, 4, 136, null, null, 1, 0, g128, null, null, null) == 1
    bad = moe.binding.MoeQuantConfig(5, 128, 128, 128)
    assert L.moe_prepare(null, 4, 128, null, null, 1, 0, ctypes.byref(bad), null, null, null) == 2
    assert L.moe_prepare(null, 4, 128, null, null, 1, 0, null, null, null, null) == 1
    assert "quant_config" in moe.last_error()


@pytest.mark.parametrize("cfg", [("fp8", 64, 128, 128), ("fp8", 128, 128, 64),
                                 ("fp8", 128, 256, 128), ("fp8_token", 128, 128, 128),
                                 ("fp8_tensor", 7, 128, 128)])
def test_prepare_rejects_unsupported_group_and_block_sizes(moe, cfg):
    """Only the G(128) group (none for per-token/per-tensor scales) and
    128x128 weight blocks are implemented; anything else is unsupported,
    reported before any launch (the pointers here are all NULL)."""
    quant, group, bn, bk = cfg
    qc = moe.binding.MoeQuantConfig(moe.binding.QUANT[quant], group, bn, bk)
    assert moe.binding.lib().moe_prepare(None, 4, 256, None, None, 1, 0, ctypes.byref(qc), None,
                                         None, None) == 2


def test_prepare_accepts_the_implemented_configs_and_ignores_topk_ids(moe):
    """The implemented configs pass validation (T == 0: a no-op that reads
    no pointer); topk_ids may be NULL or anything, it is not read."""
    L = moe.binding.lib()
    for quant in ("none", "fp8", "fp8_token", "fp8_tensor"):
        qc = moe.binding.quant_config(quant)
        assert L.moe_prepare(None, 0, 256, None, None, 1, 0, ctypes.byref(qc), None, None,
                             None) == 0
        assert L.moe_prepare(None, 0, 256, None, 12345, 1, 0, ctypes.byref(qc), None, None,
                             None) == 0
    # quant NONE ignores the group and block fields
    qc = moe.binding.MoeQuantConfig(0, 7, 3, 5)
    assert L.moe_prepare(None, 0, 256, None, None, 1, 0, ctypes.byref(qc), None, None, None) == 0


def test_validation_happens_before_any_launch_continued(moe):
    L = moe.binding.lib()
    null = None
    # align: bad block size, E too large
    assert L.moe_align(null, 4, 2, 8, 48, null, null, null, null, null, null, 0, null) == 1
    assert L.moe_align(null, 4, 2, 2000, 16, null, null, null, null, null, null, 0, null) == 1
    # finalize: fp8 output needs H % 128 == 0; negative eps
    assert L.moe_finalize(null, null, 1, null, null, null, 4, 2, 136, 0, null, null, null, null,
                          1e-6, null) == 1
    assert L.moe_finalize(null, null, 0, null, null, null, 4, 2, 128, 0, null, null, null, null,
                          -1.0, null) == 1


def test_experts_validation(moe):
    L = moe.binding.lib()
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 96, 0, 0
    # I must be a multiple of 64 (bf16 SiLU-mul)
    assert L.moe_experts(None, None, None, None, 4, 128, 2, ctypes.byref(w), 0, None, None, None, 16,
                         None, None, None, 0, None) == 2
    w.inter = 128
    # missing weight pointers
    assert L.moe_experts(None, None, None, None, 4, 128, 2, ctypes.byref(w), 0, None, None, None, 16,
                         None, None, None, 0, None) == 1
    # fp8 takes every block_m (256-row blocks run the gated first GEMM as two
    # 128-row tiles); a missing activation scale is an argument error
    w.quant = 1
    w.w13 = w.w2 = w.w13_scale = w.w2_scale = 1
    assert L.moe_experts(1, None, None, None, 4, 128, 2, ctypes.byref(w), 0, 1, 1, 1, 256,
                         1, None, None, 0, None) == 1
    # workspace too small
    w.quant = 0
    assert L.moe_experts(1, None, None, None, 4, 128, 2, ctypes.byref(w), 0, 1, 1, 1, 16,
                         1, None, None, 0, None) == 3


def test_workspace_sizes_grow_with_tokens(moe):
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 14336, 0, 0
    a = moe.moe_forward_workspace_bytes(32, 4096, 2, w)
    b = moe.moe_forward_workspace_bytes(4096, 4096, 2, w)
    assert 0 < a < b
    # z for every padded routed row + the [T, k, H] expert output dominate
    cap, blocks = oracle.align_capacity(4096, 2, 8, 128)
    assert b >= blocks * 128 * 14336 * 2 + 4096 * 2 * 4096 * 2


def test_batched_experts_validation_and_sizes(moe):
    L = moe.binding.lib()
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 128, 0, 0
    # negative max_tokens, missing weight pointers, workspace too small
    assert L.moe_experts_batched(None, None, None, -1, 128, ctypes.byref(w), 0, 0, None, None, 0,
                                 None) == 1
    assert L.moe_experts_batched(None, None, None, 4, 128, ctypes.byref(w), 0, 0, None, None, 0,
                                 None) == 1
    w.w13 = w.w2 = 1
    assert L.moe_experts_batched(1, None, 1, 4, 128, ctypes.byref(w), 0, 16, 1, None, 0, None) == 3
    # M == 0 is a no-op before any pointer is read
    assert L.moe_experts_batched(None, None, None, 0, 128, ctypes.byref(w), 0, 0, None, None, 0,
                                 None) == 0
    # fp8 at block_m 256 passes the checks up to the workspace; E * (M + block_m) is bounded
    w.quant = 1
    w.w13_scale = w.w2_scale = 1
    assert L.moe_experts_batched(1, 1, 1, 4, 128, ctypes.byref(w), 0, 256, 1, None, 0, None) == 3
    w.quant = 0
    assert L.moe_experts_batched(1, None, 1, 1 << 28, 128, ctypes.byref(w), 0, 16, 1, None, 0,
                                 None) == 1
    # the workspace holds the schedule and z for E * ceil(M / bm) * bm rows
    a = L.moe_experts_batched_workspace_bytes(16, 128, ctypes.byref(w), 0, 16)
    b = L.moe_experts_batched_workspace_bytes(256, 128, ctypes.byref(w), 0, 16)
    assert 0 < a < b
    assert b >= 8 * 256 * (4 + 128 * 2)
    lay = moe.moe_experts_batched_workspace_layout(100, 128, w, "silu", 32)
    assert lay["rows"] == 8 * 4 * 32 and lay["sorted"] == 0 and lay["z"] >= lay["rows"] * 4
    assert lay["z_scale"] is None


def test_graph_entry_validation(moe):
    L = moe.binding.lib()
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 128, 0, 0
    null = None
    h = ctypes.c_void_p()
    args = [null, null, 4, 128, 2, 0, 1, 0, ctypes.byref(w), 0, 0, null, null, 1e-6, 0, null, null,
            null, null, 0]
    # no handle pointer; the null stream cannot be captured
    assert L.moe_forward_graph_create(*args, 1, None) == 1
    assert L.moe_forward_graph_create(*args, None, ctypes.byref(h)) == 1
    assert not h.value
    assert L.moe_forward_graph_destroy(None) == 0
    assert L.moe_forward_graph_launch(None, None) == 1


def test_one_launch_entry_validation(moe):
    """moe_forward_monolithic refuses, before any HIP call, what its one
    kernel does not cover: per-token or per-tensor fp8 activations, fp8 with
    the weight on the input, more than 512 routed rows or 512 tokens, a
    missing or short workspace (status 2 = UNSUPPORTED, 3 = WORKSPACE); its
    workspace grows with the rows and hidden size, and with fp8."""
    L = moe.binding.lib()
    fake = ctypes.c_void_p(256)           # never dereferenced on these paths
    w = moe.MoeWeights()
    w.num_experts, w.inter, w.quant, w.shared_inter = 8, 128, 0, 0
    w.w13 = w.w2 = fake

    def call(T, k, weights, ws=None, wsb=0):
        return L.moe_forward_monolithic(fake, fake, T, 128, k, 0, 1, 0, ctypes.byref(weights), 0,
                                        None, None, 1e-6, 0, fake, None, None, ws, wsb, None)
    assert call(0, 2, w) == 0                      # no tokens: nothing to do
    assert call(257, 2, w) == 2                    # 514 rows
    assert call(513, 1, w) == 2                    # 513 tokens
    assert call(4, 2, w) == 3                      # no workspace
    need = L.moe_forward_monolithic_workspace_bytes(4, 128, 2, ctypes.byref(w), 0)
    assert call(4, 2, w, fake, need - 1) == 3
    assert need < L.moe_forward_monolithic_workspace_bytes(8, 128, 2, ctypes.byref(w), 0)
    assert need < L.moe_forward_monolithic_workspace_bytes(4, 256, 2, ctypes.byref(w), 0)
    f = moe.MoeWeights()
    f.num_experts, f.inter, f.quant, f.shared_inter = 8, 128, moe.binding.QUANT["fp8_token"], 0
    f.w13 = f.w2 = f.w13_scale = f.w2_scale = fake
    assert call(4, 2, f) == 2                      # per-token fp8 activations
    f.quant = moe.binding.QUANT["fp8"]
    assert call(4, 2, f) == 3                      # fp8 G(128): taken (no workspace here)
    assert L.moe_forward_monolithic(fake, fake, 4, 128, 1, 0, 1, 1, ctypes.byref(f), 0, None,
                                    None, 1e-6, 0, fake, None, None, None, 0, None) == 2
    assert (L.moe_forward_monolithic_workspace_bytes(4, 128, 2, ctypes.byref(f), 0)
            > L.moe_forward_monolithic_workspace_bytes(4, 128, 2, ctypes.byref(w), 0))
