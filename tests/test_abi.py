"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before launching anything."""

import ctypes
import os
import re

import pytest

from matrix_optimizers_sharded_amd import binding
from matrix_optimizers_sharded_amd.binding import MoMatrix, MoNsParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "matopt.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libmatopt.so is not built (python -m matrix_optimizers_sharded_amd.build)")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("muon_step_batched", "ns_orthogonalize", "sign_pack", "sign_vote"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version(lib):
    text = open(HEADER).read()
    assert lib.mo_version() == int(re.search(r"#define MATOPT_VERSION (\d+)", text).group(1))


def mats(*shapes):
    arr = (MoMatrix * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols = r, c
    return arr


def test_workspace_bytes_grows_with_padded_shapes(lib):
    one = lib.muon_workspace_bytes(mats((256, 256)), 1, binding.MO_BF16)
    # X x2 (ping-pong), A, B at 256 x 256 bf16 (k-blocked, unpadded), plus tables
    assert 4 * 256 * 256 * 2 <= one < 4 * 256 * 256 * 2 + 8192
    # a 1x1 matrix pads to 256x256
    assert lib.muon_workspace_bytes(mats((1, 1)), 1, binding.MO_BF16) == one
    assert lib.muon_workspace_bytes(mats((256, 256)), 1, binding.MO_F32) > one
    two = lib.muon_workspace_bytes(mats((256, 256), (300, 700)), 2, binding.MO_BF16)
    assert two > one
    assert lib.muon_workspace_bytes(mats((0, 5)), 1, binding.MO_BF16) == 0
    assert b"rows and cols" in lib.mo_last_error()


def test_invalid_arguments_fail_before_launch(lib):
    ns = MoNsParams(3.4445, -4.775, 2.0315, 5, 1e-7)
    fake = ctypes.c_void_p(0x1000)
    m = mats((4, 4))
    m[0].grad, m[0].momentum, m[0].out = 0x1000, 0x1000, 0x2000
    # negative iteration count
    bad = MoNsParams(1, 1, 1, -1, 1e-7)
    assert lib.muon_step_batched(m, 1, 1, 1, 1, 0.9, ctypes.byref(bad), fake, 1 << 20, None) == -1
    # unsupported dtype code
    assert lib.muon_step_batched(m, 1, 7, 1, 1, 0.9, ctypes.byref(ns), fake, 1 << 20, None) == -2
    # workspace too small / missing
    assert lib.muon_step_batched(m, 1, 1, 1, 1, 0.9, ctypes.byref(ns), fake, 16, None) == -3
    assert b"workspace too small" in lib.mo_last_error()
    assert lib.muon_step_batched(m, 1, 1, 1, 1, 0.9, ctypes.byref(ns), None, 1 << 20, None) == -3
    # missing gradient pointer
    m[0].grad = None
    assert lib.muon_step_batched(m, 1, 1, 1, 1, 0.9, ctypes.byref(ns), ctypes.c_void_p(0x100000),
                                 1 << 20, None) == -1
    # non-finite coefficient
    nan = MoNsParams(float("nan"), 1, 1, 1, 1e-7)
    assert lib.ns_orthogonalize(m, 1, 1, 1, 1, ctypes.byref(nan), fake, 1 << 20, None) == -1
    # x == out with different dtypes
    m2 = mats((4, 4))
    m2[0].x, m2[0].out = 0x100000, 0x100000
    assert lib.ns_orthogonalize(m2, 1, 1, 1, 0, ctypes.byref(ns), ctypes.c_void_p(0x200000),
                                1 << 20, None) == -1
    # count == 0 is a no-op
    assert lib.muon_step_batched(m, 0, 1, 1, 1, 0.9, ctypes.byref(ns), None, 0, None) == 0
    # sign calls
    assert lib.sign_pack(fake, 1, 0, fake, None) == -1
    assert lib.sign_pack(fake, 5, 10, fake, None) == -2
    assert lib.sign_pack(None, 1, 10, fake, None) == -1
    assert lib.sign_vote(fake, 0, 10, fake, None, None) == -1
    assert lib.sign_vote(fake, 70000, 10, fake, None, None) == -1
    assert lib.sign_vote(fake, 128, 10, fake, fake, None) == -1
    assert b"M <= 127" in lib.mo_last_error()
    assert lib.sign_vote(fake, 3, 0, fake, None, None) == -1


def test_profile_without_launches_is_empty(lib):
    assert lib.mo_profile_begin() == 0
    assert lib.mo_profile_end(None, 0) == 0


def test_size_limits_are_rejected_on_the_host(lib):
    # every padded operand buffer must stay below 2 GiB (32-bit buffer offsets)
    ok = lib.muon_workspace_bytes(mats((16384, 32768)), 1, binding.MO_BF16)
    assert ok > 2 * 16384 * 32768 * 2
    assert lib.muon_workspace_bytes(mats((32768, 32768)), 1, binding.MO_BF16) == 0
    assert b"2 GiB" in lib.mo_last_error()
    # fp32 compute doubles the element size: the same matrix that fits in bf16 does not
    assert lib.muon_workspace_bytes(mats((16384, 32768)), 1, binding.MO_F32) == 0
    assert lib.muon_workspace_bytes(mats((1 << 25, 1)), 1, binding.MO_BF16) == 0
    assert b"[1, 2^24]" in lib.mo_last_error()
    fake = ctypes.c_void_p(0x1000)
    assert lib.sign_pack(fake, 1, 1 << 45, fake, None) == -1
    assert b"too large" in lib.mo_last_error()
    assert lib.sign_unpack(fake, 1 << 45, 1, fake, None) == -1
    assert lib.sign_apply(fake, 1 << 45, 1, fake, ctypes.c_float(0.1), None) == -1


def test_next_row_calls_validate_arguments(lib):
    fake = ctypes.c_void_p(0x1000)
    ns = MoNsParams(3.4445, -4.775, 2.0315, 5, 1e-7)
    m = mats((4, 4))
    m[0].grad, m[0].momentum, m[0].out = 0x1000, 0x2000, 0x3000
    assert lib.muon_step_apply(m, 1, 1, 1, 1, 0.9, ctypes.byref(ns), ctypes.c_float(float("inf")), fake,
                               1 << 20, None) == -1
    assert b"lr" in lib.mo_last_error()
    assert lib.muon_step_apply(m, 1, 1, 1, 5, 0.9, ctypes.byref(ns), ctypes.c_float(0.1), fake, 1 << 20,
                               None) == -2
    assert lib.muon_step_apply(m, 0, 1, 1, 1, 0.9, ctypes.byref(ns), ctypes.c_float(0.1), None, 0, None) == 0
    assert lib.sign_unpack(fake, 0, 1, fake, None) == -1
    assert lib.sign_unpack(fake, 10, 3, fake, None) == -2
    assert lib.sign_unpack(None, 10, 1, fake, None) == -1
    assert lib.sign_apply(fake, 10, 1, None, ctypes.c_float(0.1), None) == -1
    assert lib.sign_apply(fake, 10, 1, fake, ctypes.c_float(float("nan")), None) == -1


def test_noalloc_rejects_lists_beyond_its_scratch_on_the_host(lib):
    """The allocation-free step checks its scratch bound on the host, before any
    HIP call: two 4096^2 matrices in bf16 need more than MO_NOALLOC_SCRATCH_BYTES."""
    ns = MoNsParams(3.4445, -4.775, 2.0315, 5, 1e-7)
    m = mats((4096, 4096), (4096, 4096))
    for i in range(2):
        m[i].grad, m[i].momentum, m[i].out = 0x1000, 0x2000, 0x3000
    need = lib.muon_workspace_bytes(m, 2, binding.MO_BF16)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert lib.muon_step_batched_noalloc(m, 2, 1, 1, 1, 0.9, ctypes.byref(ns), None) == -3
    assert b"allocation-free" in lib.mo_last_error()
    text = open(HEADER).read()
    assert re.search(r"#define MO_NOALLOC_SCRATCH_BYTES \(\(size_t\)256 << 20\)", text)
    assert binding.NOALLOC_SCRATCH_BYTES == 256 << 20


def test_sign_pack_batched_validates_on_the_host(lib):
    fake = ctypes.c_void_p(0x1000)
    out = ctypes.c_void_p(0x2000)
    assert lib.sign_pack_batched(fake, 0, 0, 64, 64, out, None) == -1            # M < 1
    assert lib.sign_pack_batched(fake, 0, 2, 64, 63, out, None) == -1            # rows overlap
    assert b"u_stride" in lib.mo_last_error()
    assert lib.sign_pack_batched(fake, 0, 2, 0, 64, out, None) == -1             # numel < 1
    assert lib.sign_pack_batched(None, 0, 2, 64, 64, out, None) == -1            # null input
    assert lib.sign_pack_batched(fake, 5, 2, 64, 64, out, None) == -2            # dtype
