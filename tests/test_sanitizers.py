"""Sanitizer runs of the host code on the CPU (no GPU involved).

- The oracle, compiled with -fsanitize=address,undefined, driven over edge-case inputs
  by tests/oracle_sanitize_driver.c (every function, exactly sized buffers, leak
  detection on).
- The oracle's own pins (tests/test_oracle_*.py except the mutation tests), run in a
  subprocess against an -fsanitize=undefined build of the oracle selected with
  ORACLE_LIB; undefined behaviour aborts the subprocess.
- The library's host-side plan construction (plan.hip, host pass compiled with
  -fsanitize=address,undefined) driven by tests/plan_sanitize_driver.cpp over random
  and adversarial chunk and tensor tables.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE_SRC = os.path.join(ROOT, "oracle", "onebit_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_oracle_under_address_and_undefined_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_san")
        subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", *SAN, "-o", exe,
                        os.path.join(HERE, "oracle_sanitize_driver.c"), ORACLE_SRC, "-lm"], check=True)
        _run(exe)


def test_oracle_pins_against_an_undefined_sanitizer_build():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_ubsan.so")
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                        "-fsanitize=undefined", "-fno-sanitize-recover=all", "-o", lib, ORACLE_SRC, "-lm"], check=True)
        pins = sorted(f for f in os.listdir(HERE) if f.startswith("test_oracle_") and f != "test_oracle_mutants.py")
        env = dict(ENV, ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", *[os.path.join(HERE, f)
                            for f in pins]], cwd=ROOT, capture_output=True, text=True, env=env, timeout=900)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
        assert "runtime error" not in r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc is not installed")
def test_plan_host_tables_under_address_and_undefined_sanitizers():
    csrc = os.path.join(ROOT, "error_compensated_bit_amd", "csrc")
    host_san = [a for f in SAN for a in ("-Xarch_host", f)]
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "plan_san")
        r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-std=c++17", *host_san, "-I", os.path.join(ROOT, "include"),
                            "-I", csrc, os.path.join(csrc, "plan.hip"), "-x", "c++",
                            os.path.join(HERE, "plan_sanitize_driver.cpp"), "-o", exe],
                           capture_output=True, text=True, cwd=d)
        assert r.returncode == 0, r.stderr[-3000:]
        _run(exe)
