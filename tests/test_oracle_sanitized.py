"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only) and run over every
function on small inputs by tests/oracle_sanitize_main.c: no out-of-bounds access, leak or undefined
behaviour in the checker the GPU parity tests rely on."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-fast-math", "-ffp-contract=off", "-Wall",
               os.path.join(HERE, "oracle_sanitize_main.c"), "-lm", "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitizer run: ok" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
