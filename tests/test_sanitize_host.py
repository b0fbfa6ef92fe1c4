"""Sanitizer builds of the host planner and argument validator (no GPU).

fa_plan.cpp is plain C++: every launch plan and argument check of the C ABI
runs there before any HIP call.  tests/sanitize/plan_sanitize.cpp drives it
over ordinary, boundary and overflowing shapes and from several threads;
this test compiles the two with g++ under AddressSanitizer +
UndefinedBehaviorSanitizer (any error aborts the run) and, separately, under
ThreadSanitizer for the concurrent calls.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefill_attention_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "plan_sanitize.cpp")
GXX = shutil.which("g++")

pytestmark = pytest.mark.skipif(GXX is None, reason="g++ is not installed")


def _build_and_run(tmp_path, sanitize: str, *args: str) -> subprocess.CompletedProcess:
    exe = str(tmp_path / f"plan_{sanitize.replace(',', '_')}")
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={sanitize}",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "fa_plan.cpp"), DRIVER, "-o", exe, "-pthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TSAN_OPTIONS="halt_on_error=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)


def test_planner_under_asan_ubsan(tmp_path):
    r = _build_and_run(tmp_path, "address,undefined")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "plan_sanitize: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planner_threads_under_tsan(tmp_path):
    r = _build_and_run(tmp_path, "thread", "threads")
    if r.returncode != 0 and "unexpected memory mapping" in r.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory on this kernel")
    assert r.returncode == 0, r.stderr[-4000:]
    assert "plan_sanitize: ok" in r.stdout
    assert "WARNING: ThreadSanitizer" not in r.stderr
