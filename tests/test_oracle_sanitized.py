"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is rebuilt with both sanitizers (out-of-bounds reads and writes,
use after free, signed overflow, misaligned or null accesses abort the run)
and the oracle pins run against that build in a child process, with the
ASan runtime loaded first as it requires.  Every entry point of the oracle
(prefill, decode step, multi-token decode, the per-channel decay, prologue,
output norm and gate) is exercised by the pins, on empty, ragged and packed
inputs.
"""
import os
import subprocess
import sys

import pytest

import oracle

TESTS = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set here; the ASan runtime has to load first")
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", *san,
                    "-Wall", "-Wextra", "-o", lib, oracle._SRC, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, RDA_ORACLE_LIB=lib, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           os.path.join(TESTS, "test_oracle_pins.py")]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900, cwd=TESTS)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, f"sanitized oracle pins failed (rc {r.returncode}):\n{tail}"
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
