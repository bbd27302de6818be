"""Build tests/c_abi/abi_step, a plain C++ caller of libmatopt.so (HIP runtime only, no
device code of its own), in-tree with hipcc; it finds the library through an rpath
relative to itself."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_step.cpp")
BIN = os.path.join(HERE, "abi_step")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose=False):
    libdir = os.path.join(ROOT, "matrix_optimizers_sharded_amd", "lib")
    rpath = os.path.relpath(libdir, HERE)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), SRC,
           "-L", libdir, "-lmatopt", f"-Wl,-rpath,$ORIGIN/{rpath}", "-o", BIN + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building tests/c_abi/abi_step")
    os.replace(BIN + ".tmp", BIN)
    if verbose:
        print(f"built {BIN}")
    return BIN


if __name__ == "__main__":
    build(verbose=True)
