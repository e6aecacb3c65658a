"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code
only) and driven over every entry point on small ragged inputs by tests/oracle_sanitize_main.c:
any out-of-bounds access or undefined behaviour in the checker aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wno-unknown-pragmas",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "fp8_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           "-lm", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "oracle sanitize: ok" in r.stdout
