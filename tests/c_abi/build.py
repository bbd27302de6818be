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


ASAN_SRC = os.path.join(HERE, "asan_host.cpp")
ASAN_LIB = os.path.join(HERE, "libmatopt_asan.so")
ASAN_BIN = os.path.join(HERE, "asan_host")
HOST_CLANG = os.environ.get("HOST_CLANGXX", "/opt/rocm/llvm/bin/clang++")


def build_asan(verbose=False):
    """A debug build of libmatopt.so whose host code (the C ABI, argument checks,
    planning, the planner) carries AddressSanitizer, and tests/c_abi/asan_host, a
    host-only program linked against it and built with the same compiler's
    sanitizer runtime.  Device code is built as usual; the sanitizer is asked for on
    the host side only."""
    src = os.path.join(ROOT, "matrix_optimizers_sharded_amd", "csrc", "matopt.hip")
    lib_cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"), "-o", ASAN_LIB + ".tmp", src]
    bin_cmd = [HOST_CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer",
               "-I", os.path.join(ROOT, "include"), ASAN_SRC, "-L", HERE, "-lmatopt_asan",
               "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib", "-L/opt/rocm/lib", "-lamdhip64",
               "-o", ASAN_BIN + ".tmp"]
    for cmd, tmp, final in ((lib_cmd, ASAN_LIB + ".tmp", ASAN_LIB), (bin_cmd, ASAN_BIN + ".tmp", ASAN_BIN)):
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"building {os.path.basename(final)} failed")
        os.replace(tmp, final)
    if verbose:
        print(f"built {ASAN_LIB} and {ASAN_BIN}")
    return ASAN_BIN


if __name__ == "__main__":
    build(verbose=True)
    if "--asan" in sys.argv:
        build_asan(verbose=True)
