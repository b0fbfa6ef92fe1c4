"""Build libfa_prefill.so in-tree for gfx950 with hipcc.

    python -m prefill_attention_amd.build        # or __graft_entry__.build()

The HIP translation units (the attention's host launcher, one kernel unit per
head dimension, the K/V producer) are compiled for gfx950 only, in parallel;
the planner is plain C++.  Packed-FP32 VALU forms are disabled for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_prefill.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa_prefill.so)")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


HIP_SOURCES = ("fa_prefill.hip", "fa_prefill_hd64.hip", "fa_prefill_hd128.hip", "fa_prefill_hd256.hip",
               "fa_kv_store.hip")


def build(verbose_resources: bool = False) -> str:
    """Compile the library; return its path."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
    plan_o = os.path.join(BUILD_DIR, "fa_plan.o")
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("a host C++ compiler (g++) is required")
    dev_flags = [
        f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=fast",
    ]
    if verbose_resources:
        dev_flags += ["-Rpass-analysis=kernel-resource-usage"]
    jobs = [[cxx, *common, "-c", os.path.join(CSRC, "fa_plan.cpp"), "-o", plan_o]]
    objs = [plan_o]
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append([hipcc, *common, *dev_flags, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, cmd) for cmd in jobs]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose_resources="-v" in sys.argv)
