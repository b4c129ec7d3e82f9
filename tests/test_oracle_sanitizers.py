"""The CPU oracle and the brute-force encoder helper built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer (host code only) and run
through tests/helpers/sanitize_main.c: ragged quantize/dequantize sizes, the
linear forward, input gradient and LoRA gradients, and a strided brute-force
encoder pass. Any out-of-bounds access, leak or undefined behaviour aborts the
run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "sanitize_main")
    src = os.path.join(HERE, "helpers", "sanitize_main.c")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", src, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized oracle checks: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
