"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m matrix_optimizers_sharded_amd.profsummary trace <stats.csv> <out.txt> --cmd "<command>"
    python -m matrix_optimizers_sharded_amd.profsummary pmc <fetch.csv> <write.csv> <out.txt> \
        --cmd-fetch "<command>" --cmd-write "<command>" [--copy-bytes N] [--by-size]
    python -m matrix_optimizers_sharded_amd.profsummary mfma <counters.csv> <out.txt> --cmd "<command>"

`mfma` summarises a `--pmc MfmaUtil MfmaFlopsBF16` run (MFMA busy share and counted
bf16 flops per dispatch).  `trace` summarises a `--kernel-trace --stats` run (calls and mean duration per
kernel kind).  `pmc` summarises two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a
command that also performs one plain device copy of --copy-bytes (bench.py
--calibrate-copy): each counter is scaled by what it reads for that copy, giving
HBM bytes per dispatch.  Both record a hash of the library's GPU code objects; the
benchmark reports the traffic figure only while that hash still matches.
"""

import argparse
import collections
import csv
import hashlib
import os
import re
import struct

PKG = os.path.dirname(os.path.abspath(__file__))

KINDS = [
    # Mangled and demangled names are both recognised.  The profiling commands pass
    # --mangled-kernels: rocprofv3's demangler turns some bf16 instantiations into
    # text that no longer shows their template arguments.
    (re.compile(r"k_ns_(gemm|small)(I.*Li0E|<[^,]+, 0,)"), "ns_syrk"),
    (re.compile(r"k_ns_(gemm|small)(I.*Li1E|<[^,]+, 1,)"), "ns_poly"),
    (re.compile(r"k_ns_(gemm|small)(I.*Li[234]E|<[^,]+, [234],)"), "ns_apply"),
    (re.compile(r"k_store_descs"), "store_descs"),
    (re.compile(r"k_momentum_sumsq"), "momentum_sumsq"),
    (re.compile(r"k_momentum_prep"), "momentum_prep"),
    (re.compile(r"k_prep_redo"), "prep_operand"),
    (re.compile(r"k_norm_scale"), "norm_scale"),
    (re.compile(r"k_scaled_copy"), "scaled_copy"),
    (re.compile(r"k_sign_pack"), "sign_pack"),
    (re.compile(r"k_sign_vote"), "sign_vote"),
    (re.compile(r"k_sign_unpack"), "sign_unpack"),
    (re.compile(r"k_sign_apply"), "sign_apply"),
    (re.compile(r"__amd_rocclr_copyBuffer"), "device_copy"),
]


def _elf_section(data, wanted):
    """Bytes of the section named `wanted` in a little-endian ELF64 image, or None."""
    if data[:4] != b"\x7fELF" or data[4] != 2 or data[5] != 1:
        return None
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):   # sh_name, sh_type, sh_flags, sh_addr, sh_offset, sh_size, ...
        return struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)

    names = header(shstrndx)[4]
    for i in range(shnum):
        h = header(i)
        start = names + h[0]
        if data[start:data.index(b"\0", start)] == wanted:
            return data[h[4]:h[4] + h[5]]
    return None


def code_hash(lib=None):
    """sha256 of the GPU code objects (the .hip_fatbin section) of the built library:
    it changes when the device code does, not when only comments or host code do."""
    from matrix_optimizers_sharded_amd.binding import library_path
    with open(lib or library_path(), "rb") as f:
        sec = _elf_section(f.read(), b".hip_fatbin")
    if sec is None:
        raise RuntimeError("no .hip_fatbin section in the library")
    return hashlib.sha256(sec).hexdigest()[:16]


# a kernel of this library (namespace mo, mangled or not); other kernels (torch's
# input generation, runtime copies) are left out of the summaries
_OWN = re.compile(r"(_ZN2mo|\bmo::)")


def kind_of(name):
    for pat, kind in KINDS:
        if pat.search(name):
            return kind
    if _OWN.search(name):
        raise ValueError(f"library kernel of no known kind: {name!r}")
    return None


def summarize_trace(stats_csv, cmd):
    calls = collections.Counter()
    total = collections.Counter()
    for r in csv.DictReader(open(stats_csv)):
        k = kind_of(r["Name"])
        if k is None:
            continue
        calls[k] += int(r["Calls"])
        total[k] += float(r["TotalDurationNs"])
    lines = [
        "# rocprofv3 --kernel-trace --stats summary, per kernel kind",
        f"# command: {cmd}",
        f"code_sha256 = {code_hash()}",
        f"{'kind':<16} {'calls':>7} {'mean_ms':>10} {'total_ms':>10}",
    ]
    for k in sorted(calls, key=lambda k: -total[k]):
        lines.append(f"{k:<16} {calls[k]:>7} {total[k] / calls[k] / 1e6:>10.4f} {total[k] / 1e6:>10.3f}")
    return "\n".join(lines) + "\n"


def _counter_by_kind(path, counter, by_size=False):
    """Counter values per kernel kind (or per kind and grid size, as kind@grid)."""
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = kind_of(r["Kernel_Name"])
        if k is None:
            continue
        if by_size and k != "device_copy":
            k = f"{k}@{r['Grid_Size']}"
        vals[k].append(float(r["Counter_Value"]))
    return vals


def summarize_pmc(fetch_csv, write_csv, cmd_fetch, cmd_write, copy_bytes, by_size=False):
    fetch = _counter_by_kind(fetch_csv, "FETCH_SIZE", by_size)
    write = _counter_by_kind(write_csv, "WRITE_SIZE", by_size)
    if "device_copy" not in fetch or "device_copy" not in write:
        raise SystemExit("no device copy dispatch found for calibration")
    # the runtime may split the calibration copy into several dispatches: sum them
    cf, cw = sum(fetch["device_copy"]), sum(write["device_copy"])
    fs = copy_bytes / (cf * 1024.0)
    ws = copy_bytes / (cw * 1024.0)
    lines = [
        "# HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per",
        "# dispatch), each scaled by what the same counter reads for one plain device copy of",
        f"# {copy_bytes} bytes in the same run" + ("; rows are kind@grid size (work-items)" if by_size else ""),
        f"# command (fetch): {cmd_fetch}",
        f"# command (write): {cmd_write}",
        f"code_sha256 = {code_hash()}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {cf:.1f}",
        f"copy_write_kib = {cw:.1f}",
        f"fetch_scale = {fs:.4f}",
        f"write_scale = {ws:.4f}",
        f"{'kind':<16} {'dispatches':>10} {'fetch_kib':>14} {'write_kib':>14} {'hbm_bytes_per_launch':>22}",
    ]
    for k in sorted(set(fetch) & set(write)):
        if k == "device_copy":
            continue
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write[k]) / len(write[k])
        b = f * 1024.0 * fs + w * 1024.0 * ws
        lines.append(f"{k:<16} {len(fetch[k]):>10} {f:>14.1f} {w:>14.1f} {b:>22.4e}")
    return "\n".join(lines) + "\n"


SIMDS = 1024                                   # 256 CUs x 4 SIMDs
BF16_FLOP_PER_SIMD_CYCLE = 2.5e15 / (SIMDS * 2.4e9)   # dense bf16 MFMA peak at 2.4 GHz


def summarize_mfma(path, cmd):
    """MfmaUtil (MFMA busy cycles / (active cycles x SIMDs)) and MfmaFlopsBF16 per
    dispatch, per kernel kind; the clock they imply is the counted flop rate over
    busy SIMD-cycles at the dense bf16 rate."""
    disp = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        k = kind_of(r["Kernel_Name"])
        if k is None or r["Counter_Name"] not in ("MfmaUtil", "MfmaFlopsBF16"):
            continue
        d = disp[r["Dispatch_Id"]]
        d["kind"] = k
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    per = collections.defaultdict(list)
    for d in disp.values():
        if "MfmaUtil" in d and "MfmaFlopsBF16" in d:
            per[d["kind"]].append(d)
    lines = [
        "# MFMA utilisation per kernel kind from rocprofv3 --pmc MfmaUtil MfmaFlopsBF16",
        "# (MfmaUtil = MFMA busy cycles / (GPU active cycles x SIMDs); MfmaFlopsBF16 = 512 x",
        "# SQ_INSTS_VALU_MFMA_MOPS_BF16); durations are those of the counter run",
        f"# command: {cmd}",
        f"code_sha256 = {code_hash()}",
        f"{'kind':<16} {'dispatches':>10} {'mfma_util_%':>11} {'bf16_flop':>12} {'ms':>9} {'TFLOP/s':>9} {'clock_GHz':>9}",
    ]
    for k in sorted(per, key=lambda k: -sum(d["MfmaFlopsBF16"] for d in per[k])):
        ds = per[k]
        util = sum(d["MfmaUtil"] for d in ds) / len(ds)
        flop = sum(d["MfmaFlopsBF16"] for d in ds) / len(ds)
        ns = sum(d["ns"] for d in ds) / len(ds)
        rate = flop / (ns * 1e-9) if ns > 0 else 0.0
        clock = rate / (util / 100.0 * SIMDS * BF16_FLOP_PER_SIMD_CYCLE) / 1e9 if util > 0 else 0.0
        lines.append(f"{k:<16} {len(ds):>10} {util:>11.2f} {flop:>12.4e} {ns / 1e6:>9.3f} {rate / 1e12:>9.1f} {clock:>9.3f}")
    return "\n".join(lines) + "\n"


def read_traffic(path, kind):
    """(bytes per launch, source hash) for `kind` from a pmc summary, or (None, None)."""
    if not os.path.exists(path):
        return None, None
    h, val = None, None
    for line in open(path):
        if line.startswith("code_sha256"):
            h = line.split("=")[1].strip()
        parts = line.split()
        if parts and parts[0] == kind and len(parts) == 5:
            val = float(parts[4])
    return val, h


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--cmd", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("fetch_csv")
    p.add_argument("write_csv")
    p.add_argument("out")
    p.add_argument("--cmd-fetch", required=True)
    p.add_argument("--cmd-write", required=True)
    p.add_argument("--copy-bytes", type=int, default=1 << 30)
    p.add_argument("--by-size", action="store_true", help="one row per kernel kind and grid size")
    m = sub.add_parser("mfma")
    m.add_argument("counter_csv")
    m.add_argument("out")
    m.add_argument("--cmd", required=True)
    a = ap.parse_args()
    if a.mode == "trace":
        text = summarize_trace(a.stats_csv, a.cmd)
    elif a.mode == "mfma":
        text = summarize_mfma(a.counter_csv, a.cmd)
    else:
        text = summarize_pmc(a.fetch_csv, a.write_csv, a.cmd_fetch, a.cmd_write, a.copy_bytes, a.by_size)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
