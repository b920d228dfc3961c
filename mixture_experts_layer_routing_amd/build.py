"""Build libmoe.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python mixture_experts_layer_routing_amd/build.py [--jobs N]
Every call recompiles every source (it is also the "does it build" check).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["route.hip", "prepare.hip", "align.hip", "finalize.hip", "splitk.hip", "batched.hip",
           "gemm_bf16.hip", "gemm_fp8.hip", "monolithic.hip", "moe_api.cpp"]

ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # no packed-fp32 instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unknown-warning-option"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{err}")
    return obj, err


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, e in results:
            if e.strip():
                print(e, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    # A kernel whose host-side stub was dropped (e.g. a device-only builtin in
    # a kernel body) links fine but fails at dlopen: refuse such a library.
    nm = shutil.which("nm") or "/usr/bin/nm"
    r = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("undefined kernel stubs in libmoe.so:\n" + "\n".join(missing[:5]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
