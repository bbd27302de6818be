"""Build libmatopt.so in-tree for gfx950 with hipcc (cross-compiles without a GPU).

    python -m matrix_optimizers_sharded_amd.build [--verbose]
"""

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "matopt.hip")
LIB = os.path.join(PKG, "lib", "libmatopt.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False, extra=()):
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, SRC]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmatopt.so")
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(res.stderr)
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
