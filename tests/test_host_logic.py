"""Host-side logic that needs no GPU: workload definitions and seeded inputs, the
benchmark's work accounting, the profile summariser, and the rule that the product
path never touches the oracle."""

import ast
import os
import textwrap

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd import workloads as W
from matrix_optimizers_sharded_amd import profsummary

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "matrix_optimizers_sharded_amd")


def test_workload_sizes():
    assert W.WORKLOADS[1].numel == 256 * 128
    assert W.WORKLOADS[2].count == 72 and W.WORKLOADS[2].numel == 84934656
    assert W.WORKLOADS[3].count == 112 and W.WORKLOADS[3].numel == 822083584
    assert W.WORKLOADS[4].count == 224 and W.WORKLOADS[4].numel == 6476005376
    assert W.WORKLOADS[5].count == 8 and W.WORKLOADS[5].shapes[0] == (4096, 4096)
    # listing order is layer-major: layer 0's seven matrices first
    assert W.WORKLOADS[4].shapes[:7] == [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]


def test_bf16_cast_is_round_to_nearest_even():
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * np.float32(1e-2)
    # include exact ties: values halfway between two bf16 numbers
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(x), want)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(want), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_host_inputs_are_seeded_and_shaped():
    a = W.host_matrix(2, 5)
    b = W.host_matrix(2, 5)
    assert a["shape"] == (3072, 768) and a["grad"].shape == (3072, 768)
    np.testing.assert_array_equal(a["grad"], b["grad"])
    np.testing.assert_array_equal(a["mom"], b["mom"])
    assert a["grad_bits"].dtype == np.uint16
    np.testing.assert_array_equal(W.bf16_bits_to_f32(a["grad_bits"]), a["grad"])
    c = W.host_matrix(2, 6)
    assert not np.array_equal(a["grad"][:768], c["grad"][:768])
    assert abs(float(a["grad"].std()) - 0.02) < 1e-3


def test_heavy_tail_rows():
    rows = W.heavy_tail_rows(3, 6, 5632)
    assert len(rows) == 56 and len(set(rows.tolist())) == 56
    d = W.host_matrix(3, 6)
    norms = np.linalg.norm(d["grad"], axis=1)
    mask = np.zeros(5632, bool)
    mask[rows] = True
    assert norms[mask].min() > 5 * norms[~mask].max() / 2


def test_bench_flop_accounting_matches_oracle_formula():
    import bench
    shapes = W.WORKLOADS[4].shapes
    f = bench.ns_flops(shapes, 5)
    total = sum(oracle.ns_polynomial_flops(r, c, 5) for r, c in shapes)
    assert sum(f.values()) == total
    assert abs(total - 4.7485e14) / 4.7485e14 < 1e-3
    b = bench.hbm_bytes(shapes, 2, 2)
    assert b["momentum_sumsq"] == W.WORKLOADS[4].numel * 10
    assert b["momentum_prep"] == W.WORKLOADS[4].numel * 12   # + write bf16 X


def test_profsummary_round_trip(tmp_path):
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    hdr = "Kernel_Name,Counter_Name,Counter_Value\n"
    fetch.write_text(hdr + textwrap.dedent("""\
        __amd_rocclr_copyBuffer,FETCH_SIZE,524288
        _ZN2mo9k_ns_gemmIDF16bLi2EDF16bEEvPKNS_7MatDescEiifff,FETCH_SIZE,1000
        _ZN2mo9k_ns_gemmIDF16bLi3EDF16bEEvPKNS_7MatDescEiifff,FETCH_SIZE,3000
        """))
    write.write_text(hdr + textwrap.dedent("""\
        __amd_rocclr_copyBuffer,WRITE_SIZE,1048576
        _ZN2mo9k_ns_gemmIDF16bLi2EDF16bEEvPKNS_7MatDescEiifff,WRITE_SIZE,100
        _ZN2mo9k_ns_gemmIDF16bLi3EDF16bEEvPKNS_7MatDescEiifff,WRITE_SIZE,300
        """))
    text = profsummary.summarize_pmc(str(fetch), str(write), "f", "w", 1 << 30)
    out = tmp_path / "s.txt"
    out.write_text(text)
    val, h = profsummary.read_traffic(str(out), "ns_apply")
    # fetch scale 2, write scale 1; mean of the two APPLY dispatches
    assert val == pytest.approx((2000 * 1024 * 2.0) + (200 * 1024 * 1.0))
    assert h == profsummary.code_hash()


def test_profsummary_kind_names():
    """Every kernel the library launches maps to the kind name the benchmark's per-kernel
    table, roofline and traffic lookup use (mangled names as hipcc emits them)."""
    names = {
        "_ZN2mo9k_ns_gemmIDF16bLi0EDF16bEEvPKNS_7MatDescEilifffPKf": "ns_syrk",
        "_ZN2mo9k_ns_gemmIDF16bLi1EDF16bEEvPKNS_7MatDescEilifffPKf": "ns_poly",
        "_ZN2mo9k_ns_gemmIDF16bLi2EDF16bEEvPKNS_7MatDescEilifffPKf": "ns_apply",
        "_ZN2mo9k_ns_gemmIfLi3EfEEvPKNS_7MatDescEilifffPKf": "ns_apply",
        "_ZN2mo9k_ns_gemmIDF16bLi4EDF16bEEvPKNS_7MatDescEilifffPKf": "ns_apply",
        "_ZN2mo15k_momentum_prepIDF16bDF16bLb1EEEvPKNS_7MatDescEifPd": "momentum_prep",
        "_ZN2mo16k_momentum_sumsqIDF16bLb1EEEvPKNS_7MatDescEifPd": "momentum_sumsq",
        "_ZN2mo11k_prep_redoIfDF16bEEvPKNS_7MatDescEiPKfPKii": "prep_operand",
        "_ZN2mo12k_norm_scaleEPKNS_7MatDescEPKdifPfS5_Pi": "norm_scale",
        "_ZN2mo13k_scaled_copyIfDF16bEEvPKNS_7MatDescEiPKfiif": "scaled_copy",
        "_ZN2mo11k_sign_packIfEEvPKT_lPji": "sign_pack",
        "_ZN2mo11k_sign_voteILi4ELb0EEEvPKjillPjPai": "sign_vote",
        "_ZN2mo13k_sign_unpackIDF16bEEvPKjlPT_i": "sign_unpack",
        "_ZN2mo12k_sign_applyIfEEvPKjlPT_fi": "sign_apply",
    }
    for mangled, kind in names.items():
        assert profsummary.kind_of(mangled) == kind, mangled
    # the library's own profiling records use the same kind names
    for kind in set(names.values()):
        assert kind in bench_kinds()


def test_profsummary_classifies_every_kernel_of_the_built_library():
    """Every kernel in the library's GPU code objects (its `<symbol>.kd` descriptors,
    each template instantiation included) maps to a kind, and the text rocprofv3's
    demangler makes of one bf16 instantiation is refused rather than dropped."""
    import re
    from matrix_optimizers_sharded_amd import binding
    path = binding.library_path()
    if not os.path.exists(path):
        pytest.fail("libmatopt.so is not built (python -m matrix_optimizers_sharded_amd.build)")
    data = open(path, "rb").read()
    syms = {m.decode() for m in re.findall(rb"(_ZN[0-9A-Za-z_]+)\.kd\0", data)}
    assert len(syms) > 20
    kinds = {s: profsummary.kind_of(s) for s in syms}
    assert all(kinds.values()), [s for s, k in kinds.items() if not k]
    assert {"ns_syrk", "ns_poly", "ns_apply", "momentum_prep", "sign_vote"} <= set(kinds.values())
    with pytest.raises(ValueError):
        profsummary.kind_of("void mo::k_ns_gemm<bool _Accum, int, E, bool _Accum, bool, E>"
                            "(mo::MatDesc const*, int, long, int, float, float, float, float const*)")


def bench_kinds():
    """Kind names the library's per-kernel timing reports (mo_profile_end)."""
    import re
    src = open(os.path.join(os.path.dirname(__file__), "..", "matrix_optimizers_sharded_amd", "csrc",
                            "matopt.hip")).read()
    block = src[src.index("kKindNames[] = {"):]
    block = block[:block.index("};")]
    return set(re.findall(r'"([a-z_]+)"', block))


def test_profsummary_mfma(tmp_path):
    path = tmp_path / "m.csv"
    hdr = "Dispatch_Id,Grid_Size,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    name = "_ZN2mo9k_ns_gemmIDF16bLi2EDF16bEEvPKNS_7MatDescEilifff"
    # two APPLY dispatches of 2 ms, 60% and 50% busy, 2.0e12 and 1.6e12 counted flops
    path.write_text(hdr + textwrap.dedent(f"""\
        1,65536,{name},MfmaUtil,60.0,0,2000000
        1,65536,{name},MfmaFlopsBF16,2.0e12,0,2000000
        2,65536,{name},MfmaUtil,50.0,0,2000000
        2,65536,{name},MfmaFlopsBF16,1.6e12,0,2000000
        """))
    text = profsummary.summarize_mfma(str(path), "cmd")
    row = [ln.split() for ln in text.splitlines() if ln.startswith("ns_apply")][0]
    assert row[1] == "2" and float(row[2]) == pytest.approx(55.0)
    assert float(row[3]) == pytest.approx(1.8e12, rel=1e-3)
    assert float(row[5]) == pytest.approx(900.0, rel=1e-3)          # TFLOP/s
    # 0.9e15 flop/s over 55% of 1024 SIMDs at the bf16 rate per SIMD-cycle
    want = 0.9e15 / (0.55 * 1024 * 2.5e15 / (1024 * 2.4e9)) / 1e9
    assert float(row[6]) == pytest.approx(want, rel=1e-3)


def _tiny_elf(payload):
    """A minimal little-endian ELF64 image with a .hip_fatbin section holding payload."""
    import struct
    names = b"\0.hip_fatbin\0.shstrtab\0"
    data_off = 64
    names_off = data_off + len(payload)
    shoff = (names_off + len(names) + 7) // 8 * 8
    head = bytearray(64)
    head[:6] = b"\x7fELF\x02\x01"
    struct.pack_into("<Q", head, 0x28, shoff)
    struct.pack_into("<HHH", head, 0x3A, 64, 3, 2)
    sh = lambda name, off, size: struct.pack("<IIQQQQIIQQ", name, 1, 0, 0, off, size, 0, 0, 1, 0)
    body = bytes(head) + payload + names
    body += b"\0" * (shoff - len(body))
    return body + bytes(64) + sh(1, data_off, len(payload)) + sh(13, names_off, len(names))


def test_code_hash_reads_the_fatbin_section(tmp_path):
    a, b = tmp_path / "a.so", tmp_path / "b.so"
    a.write_bytes(_tiny_elf(b"code object one"))
    b.write_bytes(_tiny_elf(b"code object two"))
    assert profsummary._elf_section(a.read_bytes(), b".hip_fatbin") == b"code object one"
    assert profsummary._elf_section(a.read_bytes(), b".text") is None
    assert profsummary.code_hash(str(a)) != profsummary.code_hash(str(b))
    # the built library has one, and its hash is stable
    assert profsummary.code_hash() == profsummary.code_hash()


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_product_code_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            p = os.path.join(dirpath, f)
            if f.endswith(".py"):
                assert "oracle" not in _imports(p), p
            if f.endswith((".hip", ".h")):
                assert "oracle" not in open(p).read().lower(), p
    # bench.py may use it only inside its CPU-baseline function
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.FunctionDef) and node.name != "cpu_baseline":
            for sub in ast.walk(node):
                if isinstance(sub, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in sub.names] if isinstance(sub, ast.Import) else [sub.module or ""]
                    assert not any(m.split(".")[0] == "oracle" for m in mods), node.name


def test_binding_rejects_tensors_on_different_devices():
    import torch
    from matrix_optimizers_sharded_amd import binding
    a = torch.zeros(4)
    assert binding._one_device([a, torch.zeros(2)], a) == torch.device("cpu")
    with pytest.raises(binding.MatoptError, match="one CUDA device"):
        binding._one_device([a], torch.zeros(4, device="meta"))
