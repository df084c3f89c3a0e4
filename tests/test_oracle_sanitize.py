"""The oracle under the address and undefined-behaviour sanitizers (CPU).

Builds efla_oracle.c with a small driver (oracle/sanitize_check.c) using gcc
with -fsanitize=address,undefined and no recovery, and runs forward, backward,
step and the coefficient under both rules on exactly sized heap buffers:
empty and one-token sequences, lengths ending in a partial recompute
segment, null initial states and state gradients, threads above the number
of sequences, s_final aliasing s0."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_check"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-pthread", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ORACLE, "efla_oracle.c"), os.path.join(ORACLE, "sanitize_check.c"), "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in r.stderr.lower():
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[-300:]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr
    assert "all oracle entry points clean" in run.stdout
