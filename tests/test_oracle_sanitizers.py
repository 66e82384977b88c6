"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): tests/oracle_sanitize_main.c calls every exported oracle function,
edge cases included, and any out-of-bounds access, use after free, leak or
undefined behaviour ends the run with a report and a non-zero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=gnu11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "iq_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "oracle sanitizer run ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-6000:]
