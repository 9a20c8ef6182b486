"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle/sanitize_main.c`` calls every exported oracle function on small
seeded inputs and checks invariants; here it is compiled with gcc together
with ``oracle/sfr_oracle.c`` under both sanitizers (host code only, no
OpenMP) and run.  Any out-of-bounds access, overflow or other undefined
operation aborts the run with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "sfr_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_main.c")]
FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
         "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_oracle_clean_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path / "oracle_sanitize")
    r = subprocess.run(["gcc", *FLAGS, *SRC, "-o", exe, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "clean" in r.stdout
