"""Build step of the HIP library: compiles csrc/*.hip for gfx950 and links
sparse_linear_layers_group_amd/libbitlinear.so in the source tree.

Flags: -O3, correctly rounded binary32 division (the activation quantiser
relies on it), no contraction of a multiply and an add into one fused
operation (the bit-exact elementwise kernels round every product; explicit
fmaf calls are unaffected), packed-fp32 code generation disabled, no
fast-math.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = ["abi.hip", "quant.hip", "gemv.hip", "gemm.hip", "bwd.hip"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"  # host pass only
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return obj, warn


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for obj, warn in results:
        objs.append(obj)
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
