"""Host-only AddressSanitizer and UndefinedBehaviorSanitizer run of the CPU
oracle (oracle/hs_oracle.c) and the input generator (synth/synth.c): both are
compiled with gcc and the sanitizers into one program with
tests/sanitize_main.c, which calls every function on small and edge-case
shapes (empty context, partial blocks, k = 0 and k >= n, windows longer than
the context, two levels with ragged tails, invalid page ids, token lists with
out-of-range entries, non-finite values to round). Any report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_main")
    cmd = ["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "sanitize_main.c"),
           os.path.join(ROOT, "oracle", "hs_oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
