"""bench.py on the host: its command line parses and refuses more than one GPU;
its counter reduction and traffic lookup (no GPU needed)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_help_parses():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "--workload" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _counter_csv(path, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


GEMM1_A = ("void moe::grouped_gemm_kernel<moe::GemmCfg<256, 128, 2, 4, 32, false, true, 0, 0, 2, "
           "128, false, false> >(moe::GemmParams)")
GEMM1_B = ("void moe::grouped_gemm_kernel<moe::GemmCfg<16, 64, 1, 4, 16, false, true, 0, 0, 2, "
           "128, false, false> >(moe::GemmParams)")
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctor_add<float> >()"


def test_counter_reduction_means_and_calibration(tmp_path):
    """The reduction averages the GEMM-1 dispatches and takes the last three
    elementwise launches as the copy calibration."""
    b = _bench_module()
    rows = [(COPY, "FETCH_SIZE", 7.0)]                       # an earlier elementwise launch
    rows += [(GEMM1_A, "FETCH_SIZE", v) for v in (100.0, 110.0, 120.0)]
    rows += [(COPY, "FETCH_SIZE", v) for v in (50.0, 52.0, 54.0)]
    rows += [(GEMM1_A, "WRITE_SIZE", 999.0)]                 # another counter: ignored
    _counter_csv(str(tmp_path / "p"), rows)
    g, c, n = b._pmc_means(str(tmp_path / "p"), "FETCH_SIZE")
    assert (g, c, n) == (110.0, 52.0, 3)


def test_counter_reduction_refuses_two_gemm1_kernels(tmp_path):
    """A pass that also ran another workload's GEMM-1 (the decode leg) is
    refused rather than averaged."""
    import pytest
    b = _bench_module()
    rows = [(GEMM1_A, "FETCH_SIZE", 100.0), (GEMM1_B, "FETCH_SIZE", 1.0)]
    rows += [(COPY, "FETCH_SIZE", 50.0)] * 3
    _counter_csv(str(tmp_path / "p"), rows)
    with pytest.raises(SystemExit, match="decode-leg none"):
        b._pmc_means(str(tmp_path / "p"), "FETCH_SIZE")


def test_traffic_is_reported_only_for_the_current_sources(tmp_path):
    """gemm1_traffic returns the recorded bytes while the record's source
    hash matches the GEMM sources, and None otherwise."""
    import json
    import types
    b = _bench_module()
    spec = types.SimpleNamespace(name="w@T1")
    path = str(tmp_path / "traffic.json")
    a = types.SimpleNamespace(traffic=path)
    assert b.gemm1_traffic(a, spec) is None                   # no record file
    json.dump({"w@T1": {"gemm1_bytes": 123, "sources_sha256": b.kernel_sources_digest()}},
              open(path, "w"))
    assert b.gemm1_traffic(a, spec) == 123
    json.dump({"w@T1": {"gemm1_bytes": 123, "sources_sha256": "0" * 64}}, open(path, "w"))
    assert b.gemm1_traffic(a, spec) is None
