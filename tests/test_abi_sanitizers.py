"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: every source compiled with the sanitizers on its
host pass only (device code unchanged), linked into a driver
(tests/abi_sanitize_driver.cpp) that runs argument validation of the entry
points, the size helpers and the grouped decode plan builder on the CPU.
No memory error, leak or undefined behaviour may appear."""
import concurrent.futures
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_library_host_code_under_sanitizers():
    from sparse_linear_layers_group_amd import build as B
    csrc = os.path.join(ROOT, "sparse_linear_layers_group_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        def comp(src):
            obj = os.path.join(d, os.path.basename(src) + ".o")
            r = subprocess.run([HIPCC] + B.CFLAGS + SAN + ["-g", "-c", src, "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return obj
        srcs = [os.path.join(csrc, f) for f in B.SOURCES]
        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            objs = list(ex.map(comp, srcs))
        drv = os.path.join(d, "driver.o")
        r = subprocess.run([HIPCC, "-std=c++17", "-O1", "-g", "-I", os.path.join(ROOT, "include")] + SAN +
                           ["-c", os.path.join(HERE, "abi_sanitize_driver.cpp"), "-o", drv],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        exe = os.path.join(d, "abi_sanitized")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950"] + SAN + objs + [drv, "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        # verify_asan_link_order=0: the environment may preload other
        # libraries ahead of the sanitizer runtime; leaks are checked in the
        # library's own frames only (the HIP runtime keeps allocations alive
        # until exit by design)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-3000:]
        assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-3000:]
        assert "ran clean" in r.stdout
