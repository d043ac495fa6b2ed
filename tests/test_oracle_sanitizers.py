"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
entry point runs on small seeded inputs (tests/oracle_asan/oracle_asan_driver.c)
in a build that stops at the first invalid access, leak or undefined
operation.  Host code only (gcc)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_is_clean_under_asan_and_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_asan_driver")
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        os.path.join(ROOT, "tests", "oracle_asan", "oracle_asan_driver.c"),
                        os.path.join(ROOT, "oracle", "ep_oracle.c"), "-lm", "-o", exe], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr, r.stderr
    assert "oracle sanitizer run: OK" in r.stdout
