"""Benchmark of the fused-MoE layer on one MI355X.

One step = one moe_forward call over one batch of synthetic inputs resident
in HBM: route -> prepare -> align -> routed GEMM-1 (+SiLU-mul) -> routed
GEMM-2 -> shared expert -> finalize.  Default workload: the Mixtral-shaped
bf16 layer (H=4096, I=14336, E=8, top-2, renormalised softmax, logits
N(0, 2)) at T=4096 tokens.

Prints ONE JSON line: tokens/s (value), TFLOP/s, per-stage times from HIP
events recorded on the launch stream, the dominant kernel's roofline
(routed GEMM-1, MFMA-bound), the layer's fraction of its roofline, a second
leg on the fp8 path (the DeepSeek-V3-shaped layer at T=8192 by default:
its own GEMM-1 roofline against the fp8 peak and the HBM floor), the
memory-bound stages' bandwidth (finalize at hidden 7168 with a cold cache,
align over 2^24 ids) and the CPU oracle timed on a bounded token sample on
this host ("cpu_baseline").
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE layer tokens/s & TFLOP/s (% MFMA peak); finalize GB/s, 1 MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral@T4096",
                    help="family@T<tokens>, e.g. mixtral@T4096, deepseek_v3@T8192, llama4@T2048")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--fp8-leg", default="deepseek_v3@T8192",
                    help="second workload timed in the same run (the fp8 path); 'none' to skip")
    ap.add_argument("--decode-leg", default="mixtral@T1",
                    help="decode-sized workload timed in the same run three ways: eager "
                         "moe_forward, its graph replay, and the one-launch layer; 'none' to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay leg (counter passes profile eager launches only)")
    ap.add_argument("--no-hbm-stages", action="store_true",
                    help="skip the finalize (hidden 7168) and align (2^24 ids) bandwidth legs")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens in the oracle's timed sample (about 10-30 s of CPU work)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch measured with rocprofv3 counters (json)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed steps, run a plain fp32 copy kernel (y = x * 1) over "
                         "BYTES bytes three times: the reference launch that scales the HBM "
                         "byte counters")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: read two rocprofv3 --pmc outputs (FETCH_SIZE, WRITE_SIZE) "
                         "of a --copy-calibration run and record the routed GEMM-1 traffic "
                         "for --workload in --traffic")
    return ap.parse_args()


# Routed GEMM-1: the grouped GEMM instantiated with A_GATHER (0) and EPI_Z (0);
# routed GEMM-2: A_ROWS (1) and EPI_OUT_ROUTED (1).
GEMM1_KERNEL_RE = r"grouped_gemm_kernel<.*GemmCfg<(-?\d+, ){5}(true|false), (true|false), 0, 0,"
GEMM2_KERNEL_RE = r"grouped_gemm_kernel<.*GemmCfg<(-?\d+, ){5}(true|false), (true|false), 1, 1,"
COPY_KERNEL_RE = r"elementwise|vectorized"


# The sources that define the grouped-GEMM kernels (GEMM-1 among them).
GEMM_SOURCES = ("gemm_bf16.hip", "gemm_fp8.hip", "gemm_impl.h", "launch.h", "moe_device.h")


def kernel_sources_digest():
    """sha256 over the sources of the grouped-GEMM kernels: counters taken on
    other GEMM code are stale (changes to other stages do not touch them)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_routing_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name not in GEMM_SOURCES:
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _pmc_means(run_dir, counter, kernel_re=GEMM1_KERNEL_RE):
    """Per-dispatch mean of one counter for one GEMM's kernels and the copy
    kernel."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    gemm1, copies, names = [], [], set()
    for fn in files:
        for r in csv.DictReader(open(fn)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if re.search(kernel_re, name):
                gemm1.append(v)
                names.add(name)
            elif re.search(COPY_KERNEL_RE, name):
                copies.append((int(r["Dispatch_Id"]), v))
    if len(names) > 1:
        # another workload's GEMM (e.g. the decode leg) ran in the same pass
        raise SystemExit(f"{counter}: {len(names)} different kernels match {kernel_re} in {run_dir}; "
                         "take the passes with --decode-leg none")
    # the calibration copies are the last three elementwise launches of the run
    copies = [v for _, v in sorted(copies)[-3:]]
    if not gemm1 or len(copies) < 3:
        raise SystemExit(f"{counter}: GEMM-1 or calibration dispatches missing in {run_dir}")
    return sum(gemm1) / len(gemm1), sum(copies) / len(copies), len(copies)


def write_traffic(a):
    spec = find_spec(a.workload)
    rec = {"kernel": "routed GEMM-1", "kernel_regex": GEMM1_KERNEL_RE,
           "sources_sha256": kernel_sources_digest()}
    total = 0.0
    g2 = {"kernel": "routed GEMM-2", "kernel_regex": GEMM2_KERNEL_RE}
    total2 = 0.0
    for counter, run_dir in (("FETCH_SIZE", a.write_traffic[0]), ("WRITE_SIZE", a.write_traffic[1])):
        g_kib, c_kib, n = _pmc_means(run_dir, counter)
        factor = c_kib * 1024.0 / a.copy_calibration     # counter bytes per true byte
        rec[counter] = {"gemm1_kib_per_dispatch": round(g_kib, 1),
                        "copy_kib_per_dispatch": round(c_kib, 1), "copy_dispatches": n,
                        "copy_true_bytes": a.copy_calibration, "factor": round(factor, 4),
                        "gemm1_bytes": round(g_kib * 1024.0 / factor)}
        total += g_kib * 1024.0 / factor
        g2_kib, _, _ = _pmc_means(run_dir, counter, GEMM2_KERNEL_RE)
        g2[counter] = {"kib_per_dispatch": round(g2_kib, 1), "factor": round(factor, 4),
                       "bytes": round(g2_kib * 1024.0 / factor)}
        total2 += g2_kib * 1024.0 / factor
    rec["gemm1_bytes"] = round(total)
    g2["bytes"] = round(total2)
    rec["gemm2"] = g2
    tr = {}
    if os.path.exists(a.traffic):
        tr = json.load(open(a.traffic))
    tr[spec.name] = rec
    with open(a.traffic, "w") as f:
        json.dump(tr, f, indent=1)
        f.write("\n")
    print(json.dumps({spec.name: rec}))


def find_spec(name):
    from workloads import CONFIGS
    for fam in CONFIGS.values():
        for s in fam:
            if s.name == name:
                return s
    raise SystemExit(f"unknown workload {name}")


def layer_flops(spec):
    """Algorithmic flops of one layer call: the selected experts only
    (2 flops per multiply-add), no padding rows."""
    g = 2 if spec.activation == "silu" else 1
    routed = 2.0 * spec.T * spec.top_k * spec.H * spec.I * (g + 1)
    shared = 2.0 * spec.T * spec.H * spec.shared_I * (g + 1)
    return routed, shared


def gemm1_flops(spec):
    g = 2 if spec.activation == "silu" else 1
    return 2.0 * spec.T * spec.top_k * spec.H * spec.I * g


def layer_roofline(spec, touched):
    """The layer's roofline time: its algorithmic flops at the dense MFMA
    peak of its dtype, or its algorithmic HBM bytes at 8 TB/s, whichever is
    longer.  Bytes: the touched experts' weights (+ fp8 block scales) and
    the shared expert's, read once; x read; a1q written and read; z written
    and read; fused_expert_output written and read; the output written.
    Padding rows are not counted."""
    fp8 = spec.quant.startswith("fp8")
    eb = 1 if fp8 else 2
    g = 2 if spec.activation in ("silu", "gelu") else 1
    H, I, Is, T, k = spec.H, spec.I, spec.shared_I, spec.T, spec.top_k
    w = touched * (g * I * H + H * I) * eb + (g * Is * H + H * Is) * eb
    if fp8:
        w += 4 * (touched * (g * I * H + H * I) + (g * Is * H + H * Is)) // (128 * 128)
    act = T * H * 2 + 2 * T * H * eb + 2 * (T * k * I + T * Is) * eb + 2 * T * k * H * 2 \
        + T * H * 2
    routed, shared = layer_flops(spec)
    t_mfma = (routed + shared) / (PEAK_TFLOPS["fp8" if fp8 else "bf16"] * 1e12)
    t_hbm = (w + act) / (PEAK_HBM_GBS * 1e9)
    return {"ms": round(max(t_mfma, t_hbm) * 1e3, 4), "bound": "mfma" if t_mfma > t_hbm else "hbm",
            "flops": routed + shared, "bytes": int(w + act), "touched_experts": int(touched)}


def cpu_baseline(spec, d, sample_n):
    import numpy as np
    import oracle
    from workloads import to_numpy_bits
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    keys = ("w13", "w13_scale", "w2", "w2_scale", "shared_w13", "shared_w13_scale", "shared_w2",
            "shared_w2_scale")
    hw = {k: to_numpy_bits(d[k]) for k in keys if d.get(k) is not None}
    x = to_numpy_bits(d["x"])
    logits = d["logits"].cpu().numpy()
    res = to_numpy_bits(d.get("residual"))
    gam = to_numpy_bits(d.get("gamma"))
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(spec.T, size=min(sample_n, spec.T), replace=False))
    t0 = time.perf_counter()
    oracle.forward(x, logits, hw, spec.top_k, spec.scoring, spec.renormalize, 16,
                   spec.apply_router_weight_on_input, spec.quant, spec.activation, "mirrored",
                   res, gam, spec.eps, spec.out_quant, tokens=sample)
    dt = time.perf_counter() - t0
    return {"value": round(sample.size / dt, 3), "unit": "tokens/s", "cores": threads,
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{sample.size} of {spec.T} tokens (route+align over all {spec.T}), "
                      f"numpy float64, mirrored mode, {dt:.1f} s; cores = BLAS threads, "
                      f"host_cpus = CPUs this process may run on"}


def hbm_stages(torch, moe, dev):
    """Memory-bound stages at the sizes where bandwidth, not launch latency,
    is what they show: finalize on the hidden-7168 fusion shape (k=4,
    shared + residual + RMSNorm, T=16384; bf16 and fp8 output) with two input
    sets of 1.6 GB alternating, so every call reads from HBM rather than the
    256 MB last-level cache; and align over 2^24 ids.  GB/s counts the bytes
    the stage must move once (algorithmic), timed with HIP events over 20
    back-to-back calls."""
    from workloads import CONFIGS, make_finalize_inputs

    def timed(fn, calls):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls   # us

    out = {}
    spec = [s for s in CONFIGS["finalize"] if s.T == 16384 and s.out_quant == "none"][0]
    sets = []
    for r in range(2):
        d = make_finalize_inputs(spec, device=dev) if r == 0 else \
            {k: (v.clone() if torch.is_tensor(v) else v) for k, v in sets[0].items()}
        sets.append(d)
    T, k, H = spec.T, spec.top_k, spec.H
    for oq in ("none", "fp8"):
        outs = [torch.empty((T, H), dtype=torch.bfloat16 if oq == "none" else torch.uint8,
                            device=dev) for _ in sets]
        scs = [torch.empty((T, H // 128), dtype=torch.float32, device=dev) for _ in sets]

        def fin(i, oq=oq, outs=outs, scs=scs):
            d = sets[i % 2]
            moe.moe_finalize(d["fused_expert_output"], d["topk_weights"], d["topk_ids"], False,
                             d["shared"], d["residual"], d["gamma"], spec.eps, oq,
                             output=outs[i % 2], output_scale=scs[i % 2] if oq == "fp8" else None)
        us = timed(fin, 20)
        per_tok = k * H * 2 + k * 4 + 2 * H * 2 + (H * 2 if oq == "none" else H + H // 128 * 4)
        gbs = T * per_tok / us / 1e3
        out["finalize" if oq == "none" else "finalize_fp8_out"] = {
            "workload": f"finalize T={T} k={k} H={H} shared+residual+RMSNorm, {oq} out, cold",
            "bytes_per_token": per_tok, "us": round(us, 2), "GB_s": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    del sets
    torch.cuda.empty_cache()
    sweep = []
    for E, kk, bm in ((8, 2, 256), (256, 8, 128)):
        # four id sets with their outputs (4 x 128 MB > the last-level cache),
        # called in rotation with preallocated outputs and workspace
        n = 1 << 24
        g = torch.Generator(device=dev)
        g.manual_seed(E)
        # top-k routing: kk distinct experts per token, uniformly at random
        idss = [torch.rand((n // kk, E), device=dev, generator=g).topk(kk, dim=1).indices
                .to(torch.int32).contiguous() for _ in range(4)]
        ress = [moe.moe_align(ids, E, bm) for ids in idss]

        def al(i, idss=idss, ress=ress, E=E, bm=bm):
            moe.moe_align(idss[i % 4], E, bm, out=ress[i % 4])
        us = timed(al, 20)
        res = ress[0]
        alg = 4 * n + 4 * (res["sorted_token_ids"].numel() + res["block_expert_ids"].numel()) \
            + 8 * E + 8
        gbs = alg / us / 1e3
        sweep.append({"n_ids": n, "E": E, "top_k": kk, "block_m": bm, "us": round(us, 2),
                      "GB_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        del idss, ress, res
    out["align_sweep"] = sweep
    return out


def measure(a, torch, moe, spec, block_m=0, graph=True):
    """Time one workload: K plain moe_forward steps (the headline), K steps
    with stage events (per-stage times, GEMM-1's duration), and K replays
    of the step as one graph launch.  Returns (result dict, inputs)."""
    from workloads import make_layer_inputs
    dev = "cuda"
    d = make_layer_inputs(spec, device=dev)
    w = moe.make_weights(*(d.get(k) for k in ("w13", "w2", "w13_scale", "w2_scale", "shared_w13",
                                              "shared_w2", "shared_w13_scale", "shared_w2_scale")))
    bm = block_m or moe.moe_pick_block_m(spec.T, spec.top_k, spec.E, spec.quant)
    stream = torch.cuda.current_stream()

    def step(events=None, ws=None, out=None):
        return moe.moe_forward(d["x"], d["logits"], w, spec.top_k, spec.scoring, spec.renormalize,
                               spec.apply_router_weight_on_input, spec.activation, bm,
                               d.get("residual"), d.get("gamma"), spec.eps, spec.out_quant,
                               output=out, workspace=ws, stage_events=events)

    out, _, ws = step()
    for _ in range(a.warmup):
        step(ws=ws, out=out)
    # the timed steps: plain moe_forward calls, nothing recorded between kernels
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(ws=ws, out=out)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / a.steps
    # the same number of steps again with an event between stages: the
    # per-stage times and the GEMM-1 duration of the roofline (the events
    # themselves add small gaps, so the step time above is taken without them)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.NUM_STAGE_EVENTS)]
           for _ in range(a.steps)]
    for i in range(a.steps):
        step(events=evs[i], ws=ws, out=out)
    torch.cuda.synchronize()
    # the same step replayed as one graph launch (moe_forward_graph_*): the
    # kernels and buffers are identical, only the per-kernel host submission
    # is gone -- the rate a decode loop sees
    graph_ms = None
    if graph:
        gstream = torch.cuda.Stream()
        with torch.cuda.stream(gstream):
            g = moe.ForwardGraph(d["x"], d["logits"], w, spec.top_k, spec.scoring,
                                 spec.renormalize, spec.apply_router_weight_on_input,
                                 spec.activation, bm, d.get("residual"), d.get("gamma"),
                                 spec.eps, spec.out_quant)
            for _ in range(a.warmup):
                g.launch(gstream)
        torch.cuda.synchronize()
        gstart, gstop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gstart.record(gstream)
        for _ in range(a.steps):
            g.launch(gstream)
        gstop.record(gstream)
        torch.cuda.synchronize()
        graph_ms = gstart.elapsed_time(gstop) / a.steps
        g.close()
        del g
    # the one-launch layer (moe_forward_monolithic), where it applies: bf16
    # weights, or fp8 with G(128) activations and no weight on the input;
    # T <= 512, T*top_k <= 512
    mono_ms = None
    fits = spec.quant == "none" or (spec.quant == "fp8" and not spec.apply_router_weight_on_input)
    if graph and fits and spec.T <= 512 and spec.T * spec.top_k <= 512:
        def mono(out_m=None, ws_m=None):
            return moe.moe_forward_monolithic(
                d["x"], d["logits"], w, spec.top_k, spec.scoring, spec.renormalize,
                spec.apply_router_weight_on_input, spec.activation, d.get("residual"),
                d.get("gamma"), spec.eps, spec.out_quant, output=out_m, workspace=ws_m)
        mout, _, mws = mono()
        for _ in range(a.warmup):
            mono(mout, mws)
        torch.cuda.synchronize()
        mstart, mstop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mstart.record(stream)
        for _ in range(a.steps):
            mono(mout, mws)
        mstop.record(stream)
        torch.cuda.synchronize()
        mono_ms = mstart.elapsed_time(mstop) / a.steps
        del mout, mws
    stage = {}
    for j in range(1, moe.NUM_STAGE_EVENTS):
        vals = [evs[i][j - 1].elapsed_time(evs[i][j]) for i in range(a.steps)]
        stage[moe.STAGES[j]] = sum(vals) / len(vals)
    ids, _ = moe.moe_route(d["logits"], spec.top_k, spec.scoring, spec.renormalize)
    touched = int(torch.unique(ids).numel())
    routed, shared = layer_flops(spec)
    dtype = "fp8" if spec.quant.startswith("fp8") else "bf16"
    g1_ms = stage["gemm1"]
    g1_tflops = gemm1_flops(spec) / (g1_ms * 1e-3) / 1e12
    roof = layer_roofline(spec, touched)
    res = {
        "ms": ms, "wall": wall, "bm": bm, "stage": stage, "graph_ms": graph_ms, "mono_ms": mono_ms,
        "tflops": (routed + shared) / (ms * 1e-3) / 1e12, "dtype": dtype,
        "g1_ms": g1_ms, "g1_tflops": g1_tflops, "layer_roofline": roof,
        # GEMM-1's weights streamed once: the HBM floor of that kernel
        "g1_hbm_floor_ms": touched * (2 if spec.activation in ("silu", "gelu") else 1) * spec.I
        * spec.H * (1 if dtype == "fp8" else 2) / (PEAK_HBM_GBS * 1e9) * 1e3,
    }
    return res, d, (w, out, ws)


def gemm1_traffic(a, spec):
    """GEMM-1's HBM bytes per launch from the counter record of this
    workload, or None when there is none or it was taken on other GEMM code."""
    if not os.path.exists(a.traffic):
        return None
    try:
        rec = json.load(open(a.traffic)).get(spec.name, {})
    except Exception:
        return None
    return rec.get("gemm1_bytes") if rec.get("sources_sha256") == kernel_sources_digest() else None


def _roofline(spec, res, traffic):
    dtype = res["dtype"]
    return {"kernel": "routed GEMM-1 (gate+up, SiLU-mul fused)", "bound": "mfma",
            "achieved": round(res["g1_tflops"], 2), "peak": PEAK_TFLOPS[dtype],
            "unit": "TFLOP/s", "frac": round(res["g1_tflops"] / PEAK_TFLOPS[dtype], 4),
            "traffic": traffic,
            "timing": "GEMM-1's average duration over the K instrumented steps, from HIP "
                      "events recorded on the launch stream before and after it inside "
                      "moe_forward"}


def main():
    a = parse()
    if a.write_traffic:
        if a.copy_calibration <= 0:
            raise SystemExit("--write-traffic needs --copy-calibration BYTES of the profiled run")
        write_traffic(a)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU sharding is a design note, not implemented)"}))
        sys.exit(2)
    import torch
    import mixture_experts_layer_routing_amd as moe

    spec = find_spec(a.workload)
    dev = "cuda"
    res, d, keep = measure(a, torch, moe, spec, a.block_m, graph=not a.no_graph)
    ms = res["ms"]
    traffic = gemm1_traffic(a, spec)
    roof = res["layer_roofline"]
    line = {
        "metric": METRIC,
        "value": round(spec.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        "config": {"workload": spec.name, "T": spec.T, "H": spec.H, "I": spec.I, "E": spec.E,
                   "top_k": spec.top_k, "scoring": spec.scoring, "renormalize": spec.renormalize,
                   "quant": spec.quant, "shared_I": spec.shared_I, "block_m": res["bm"],
                   "parallelism": "none (1 GPU)"},
        "tflops": round(res["tflops"], 2),
        "mfma_peak_frac": round(res["tflops"] / PEAK_TFLOPS[res["dtype"]], 4),
        "layer_roofline": dict(roof, frac=round(roof["ms"] / ms, 4)),
        "stage_ms": {k: round(v, 4) for k, v in res["stage"].items()},
        "graph": None if res["graph_ms"] is None else {
            "ms_per_step": round(res["graph_ms"], 4),
            "tokens_per_s": round(spec.T / (res["graph_ms"] * 1e-3), 1)},
        "one_launch": None if res["mono_ms"] is None else {
            "ms_per_step": round(res["mono_ms"], 4),
            "tokens_per_s": round(spec.T / (res["mono_ms"] * 1e-3), 1)},
        "wall_s": round(res["wall"], 3),
        "roofline": _roofline(spec, res, traffic),
    }
    cpu_inputs = None
    if not a.no_cpu_baseline:
        cpu_inputs = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in d.items()}
    del d, keep
    torch.cuda.empty_cache()
    if a.fp8_leg != "none" and a.fp8_leg != spec.name:
        # the fp8 path in the same run: its own roofline against the fp8 peak
        # and GEMM-1's HBM floor, and the layer's fraction of its roofline
        fspec = find_spec(a.fp8_leg)
        fres, fd, fkeep = measure(a, torch, moe, fspec, 0, graph=False)
        froof = fres["layer_roofline"]
        line["fp8_leg"] = {
            "workload": fspec.name, "ms_per_step": round(fres["ms"], 4),
            "tokens_per_s": round(fspec.T / (fres["ms"] * 1e-3), 1),
            "tflops": round(fres["tflops"], 2), "block_m": fres["bm"],
            "stage_ms": {k: round(v, 4) for k, v in fres["stage"].items()},
            "layer_roofline": dict(froof, frac=round(froof["ms"] / fres["ms"], 4)),
            "roofline": dict(_roofline(fspec, fres, gemm1_traffic(a, fspec)),
                             hbm_floor_ms=round(fres["g1_hbm_floor_ms"], 4),
                             hbm_floor_frac=round(fres["g1_hbm_floor_ms"] / fres["g1_ms"], 4)),
        }
        del fd, fkeep
        torch.cuda.empty_cache()
    if a.decode_leg != "none" and a.decode_leg != spec.name:
        # a decode step three ways: eager launches, one graph launch of the
        # same kernels, and the one-launch layer (one persistent kernel)
        dspec = find_spec(a.decode_leg)
        dres, dd_, dkeep = measure(a, torch, moe, dspec, 0, graph=True)
        line["decode_leg"] = {
            "workload": dspec.name, "block_m": dres["bm"],
            "eager_ms": round(dres["ms"], 4),
            "graph_ms": None if dres["graph_ms"] is None else round(dres["graph_ms"], 4),
            "one_launch_ms": None if dres["mono_ms"] is None else round(dres["mono_ms"], 4),
            "layer_roofline_ms": round(dres["layer_roofline"]["ms"], 4),
            "stage_ms": {k: round(v, 4) for k, v in dres["stage"].items()},
        }
        del dd_, dkeep
        torch.cuda.empty_cache()
    if not a.no_hbm_stages:
        line.update(hbm_stages(torch, moe, dev))
    if a.copy_calibration:
        # the last GPU work of the run: the counter reduction takes the last
        # three elementwise launches as the calibration copies
        n = a.copy_calibration // 4
        cx = torch.ones(n, dtype=torch.float32, device=dev)
        cy = torch.empty_like(cx)
        for _ in range(3):
            torch.mul(cx, 1.0, out=cy)
        torch.cuda.synchronize()
        del cx, cy
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, cpu_inputs, a.cpu_sample)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
