"""Build libfa_prefill.so in-tree for gfx950 with hipcc.

    python -m prefill_attention_amd.build        # or __graft_entry__.build()
    python -m prefill_attention_amd.build --kv-tile 32 --waves 4
                       # another tile geometry, for measurement, into
                       # prefill_attention_amd/geometry/kv32_w4/libfa_prefill.so

The HIP translation units (the attention's host launcher, one kernel unit per
head dimension, the K/V producer) are compiled for gfx950 only, in parallel;
the planner is plain C++.  Packed-FP32 VALU forms are disabled for the device code.
"""

from __future__ import annotations

import os
import re
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
    r = subprocess.run(cmd, capture_output=True, text=True)
    sys.stdout.write(r.stdout)
    if r.returncode:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    return r.stderr


def kernel_resources(remarks: str) -> dict:
    """Per-kernel register, scratch and occupancy figures from hipcc's
    -Rpass-analysis=kernel-resource-usage remarks: {name: {field: value}}."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[a-z/A-Z]+\])?: (\d+)", line)
        if m and cur is not None:
            out[cur][m.group(1).strip()] = int(m.group(2))
    return out


def check_resources(resources: dict) -> None:
    """Fail the build when a shipped kernel spills or uses scratch memory.

    A spill silently turns register traffic into memory traffic; like any
    resource limit of the launch it must stop the build rather than ship a
    slower kernel (the pages' rule that resource limits fail loudly).
    """
    bad = {name: r for name, r in resources.items()
           if r.get("ScratchSize", 0) or r.get("VGPRs Spill", 0) or r.get("SGPRs Spill", 0)}
    if bad:
        lines = [f"  {n}: ScratchSize={r.get('ScratchSize')} VGPRs Spill={r.get('VGPRs Spill')} "
                 f"SGPRs Spill={r.get('SGPRs Spill')}" for n, r in bad.items()]
        raise RuntimeError("kernels with register spills or scratch memory:\n" + "\n".join(lines))


HIP_SOURCES = ("fa_prefill.hip", "fa_prefill_hd64.hip", "fa_prefill_hd128.hip", "fa_prefill_hd256.hip",
               "fa_kv_store.hip")


SHIPPED_GEOMETRY = (64, 4)  # (key/value tile rows, wavefronts per work-group)


def geometry_lib_path(kv_tile: int, waves: int) -> str:
    """Where a build of another tile geometry goes by default (bench.py --lib)."""
    return os.path.join(PKG, "geometry", f"kv{kv_tile}_w{waves}", LIB_NAME)


def build(verbose_resources: bool = False, kv_tile: int = 64, waves: int = 4, out: str | None = None,
          allow_spills: bool = False) -> str:
    """Compile the library; return its path.  Fails if any kernel spills.

    kv_tile / waves select another tile geometry (FA_KV_TILE in {32, 64,
    128}, FA_WAVES in {4, 8}) for measuring it; such a build goes to `out`
    or geometry_lib_path() and never replaces the shipped library.  allow_spills lets a
    geometry whose register budget overflows build anyway (for measurement
    only; the shipped geometry never spills).
    """
    from concurrent.futures import ThreadPoolExecutor

    shipped = (kv_tile, waves) == SHIPPED_GEOMETRY
    lib_path = os.path.abspath(out) if out else (LIB_PATH if shipped else geometry_lib_path(kv_tile, waves))
    build_dir = BUILD_DIR if shipped else os.path.join(BUILD_DIR, f"kv{kv_tile}_w{waves}")
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib_path), exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
    if not shipped:
        common += [f"-DFA_KV_TILE={kv_tile}", f"-DFA_WAVES={waves}"]
    plan_o = os.path.join(build_dir, "fa_plan.o")
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        raise RuntimeError("a host C++ compiler (g++) is required")
    dev_flags = [
        f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=fast",
    ]
    dev_flags += ["-Rpass-analysis=kernel-resource-usage"]
    jobs = [[cxx, *common, "-c", os.path.join(CSRC, "fa_plan.cpp"), "-o", plan_o]]
    objs = [plan_o]
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        jobs.append([hipcc, *common, *dev_flags, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    resources = {}
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, cmd) for cmd in jobs]:
            resources.update(kernel_resources(f.result()))
    if verbose_resources:
        for name, r in sorted(resources.items()):
            print(f"{name}: {r}")
    if not (allow_spills and not shipped):
        check_resources(resources)
    tmp = lib_path + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib_path)
    if shipped:
        build_probes(hipcc, common, dev_flags)
    return lib_path


PROBE_SRC = os.path.join(ROOT, "tests", "probes", "fa_probes.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "probes", "libfa_probes.so")


def build_probes(hipcc, common, dev_flags) -> None:
    """The GPU tests' single-instruction layout probes (test infrastructure,
    not part of the library): tests/probes/libfa_probes.so."""
    if not os.path.exists(PROBE_SRC):
        return
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, *common, *[f for f in dev_flags if not f.startswith("-Rpass")], "-shared", PROBE_SRC, "-o", tmp])
    os.replace(tmp, PROBE_LIB)


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser(description="build libfa_prefill.so for gfx950")
    ap.add_argument("-v", action="store_true", help="print every kernel's register / scratch / LDS figures")
    ap.add_argument("--kv-tile", type=int, default=SHIPPED_GEOMETRY[0], help="key/value rows per tile (32, 64, 128)")
    ap.add_argument("--waves", type=int, default=SHIPPED_GEOMETRY[1], help="wavefronts per work-group (4, 8)")
    ap.add_argument("--out", default=None, help="library path (default: in-tree; another geometry: "
                                                "prefill_attention_amd/geometry/kv<T>_w<W>/)")
    ap.add_argument("--allow-spills", action="store_true", help="build a spilling non-shipped geometry anyway")
    a = ap.parse_args()
    print(build(verbose_resources=a.v, kv_tile=a.kv_tile, waves=a.waves, out=a.out, allow_spills=a.allow_spills))
