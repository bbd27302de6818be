"""The C ABI's host code under AddressSanitizer (and LeakSanitizer): a debug build of
the library whose host side is instrumented, driven by tests/c_abi/asan_host.cpp
through argument validation of every entry point, workspace sizing over random shape
lists, the owner planner and the profiling calls.  Needs no GPU: every call it makes
is rejected on the host or never touches a device.  The pair is rebuilt (about a
minute) when it is missing or older than its sources."""

import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _sources():
    return (glob.glob(os.path.join(ROOT, "matrix_optimizers_sharded_amd", "csrc", "*")) +
            [os.path.join(ROOT, "include", "matopt.h"), os.path.join(HERE, "c_abi", "asan_host.cpp"),
             os.path.join(HERE, "c_abi", "build.py")])


def test_host_abi_under_address_sanitizer():
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(HERE, "c_abi", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    for tool in (b.HIPCC, b.HOST_CLANG):
        if not (os.path.exists(tool) or shutil.which(tool)):
            pytest.skip(f"{tool} not available")
    newest = max(os.path.getmtime(p) for p in _sources())
    built = [p for p in (b.ASAN_LIB, b.ASAN_BIN) if os.path.exists(p)]
    if len(built) < 2 or min(os.path.getmtime(p) for p in built) < newest:
        b.build_asan()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1")
    res = subprocess.run([b.ASAN_BIN], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ok: 0 failure(s)" in res.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "ERROR: LeakSanitizer" not in out, out[-4000:]
