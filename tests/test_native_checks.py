"""Host-only native checks, built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU code is compiled here):

- plan_fuzz: seeded random calls of the planner (phase 1), valid and broken, with the
  work-list coverage invariants checked in C++ (tests/native/plan_fuzz.cpp);
- prefill_visit_check: the prefill kernel's key-tile visiting order, exhaustively over
  small shapes (tests/native/prefill_visit_check.cpp).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "paged_kv_cache_314_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]


def _build(tmp_path, name, sources, opt="-O1"):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", opt, *SAN, "-I", INCLUDE, "-I", CSRC, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def _run(cmd):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.parametrize("seed", [314, 2718])
def test_planner_fuzz_under_sanitizers(tmp_path, seed):
    exe = _build(tmp_path, "plan_fuzz", [os.path.join(NATIVE, "plan_fuzz.cpp"),
                                         os.path.join(CSRC, "plan.cpp")])
    out = _run([exe, "250", str(seed)])
    assert "0 failures" in out, out


def test_prefill_visit_order_exhaustive(tmp_path):
    exe = _build(tmp_path, "prefill_visit_check",
                 [os.path.join(NATIVE, "prefill_visit_check.cpp")], opt="-O2")
    out = _run([exe])
    assert "0 failures" in out, out
