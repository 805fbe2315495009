"""The oracle's pins, run once more against a build of the oracle instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no GPU).

An out-of-bounds read or write, a use after free or an undefined operation
(signed overflow, a bad shift, a misaligned access) anywhere in the oracle
aborts that run, so the pins and the randomised cases must pass without a
single report.  The child process gets the ASan runtime preloaded because the
Python interpreter itself is not instrumented; leak checking is off (the
interpreter keeps its own allocations to the end).
"""
import os
import subprocess
import sys

import pytest

from oracle.build import SAN_LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_plan.py", "tests/test_oracle_hist_reroute.py",
        "tests/test_oracle_stats_slotfill.py", "tests/test_oracle_dispatch.py",
        "tests/test_oracle_domain.py", "tests/test_oracle_grad_reduce.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set in this environment; the sanitizer runtime must come first")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's ASan runtime is not installed")
    build(sanitize=True)
    env = dict(os.environ, EP_ORACLE_LIB=SAN_LIB_PATH, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    assert " passed" in r.stdout, tail
