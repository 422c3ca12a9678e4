"""Host code under the address and undefined-behaviour sanitizers (CPU only).

* The launch planner (histogram_gradient_boosted_amd/csrc/hgb_plan.h, plain
  C++) is compiled with g++ -fsanitize=address,undefined into
  tests/host/plan_test.cpp's checks -- the workloads' shapes, random shapes,
  adversarial node lists (65,535 nodes, empty, skipped and giant nodes, level
  orders ending near 2^31) -- and run.
* The oracle is rebuilt with the same sanitizers and its own tests are run
  against that build in a child process that preloads the ASan runtime.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "histogram_gradient_boosted_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def test_planner_under_sanitizers():
    _need("g++")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "plan_test")
        subprocess.run(["g++", "-std=c++17", "-O1", *SAN, "-I", CSRC, "-o", exe,
                        os.path.join(ROOT, "tests", "host", "plan_test.cpp")], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                           env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "checks passed" in r.stdout


def test_oracle_tests_under_sanitizers():
    _need("gcc")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("the ASan runtime is not installed")
    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_"))
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
