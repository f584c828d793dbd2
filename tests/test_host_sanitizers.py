"""The host C code (the oracle and the input generator) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host/sanitize_driver.c runs every exported routine once on small
inputs and edge cases; any out-of-bounds access, leak, signed overflow or other undefined behaviour
fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "host", "sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "sanitize driver ok" in r.stdout, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
