"""The oracle built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc), every entry point driven on small seeded
inputs of all six patterns (tests/oracle_sanitize_driver.c): no memory
error, leak or undefined behaviour may appear, and the pack round trips
and paired evaluations inside the driver must hold."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_address_and_undefined_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
               "-lpthread", "-lm", "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        assert b.returncode == 0, b.stderr[-3000:]
        # verify_asan_link_order=0: the environment may preload other
        # libraries ahead of the sanitizer runtime
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
        assert "ran clean" in r.stdout
