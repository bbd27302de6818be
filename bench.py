"""Benchmark of the owner-local Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7b-class]

One step = one muon_step_batched call over the whole owner set (momentum, Frobenius
scaling, k Newton-Schulz iterations on every matrix), inputs resident in HBM.  The
sign-vote workload's step is ns_orthogonalize over the 8 worker momenta followed by
one sign_pack_batched over the 8 workers and one sign_vote.

Prints ONE JSON line: matrix params/s (value), achieved TFLOP/s and % of the dense
MFMA peak of the compute dtype, a per-kernel breakdown from HIP events recorded by
the library on the launch stream, the roofline of the dominant kernel, the same
figures for the other owner sets (other_workloads: 125M-class, 1B-class, the
Sign-Muon vote set, the single 256x128 fp32 matrix, and the 1B-class set with fp32
compute) and the fp64 CPU oracle timed on the host cores.  --blas-ceiling adds
what torch.matmul (hipBLASLt) sustains on the same product shapes.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

NAMES = {"single-256x128": 1, "125m-class": 2, "1b-class-swiglu": 3, "7b-class": 4, "sign-vote-8x4096": 5}


def ns_flops(shapes, iters):
    """Algorithmic flops per kernel kind for one step: per matrix and iteration
    m^2 n (upper triangle of X X^T), m^3 (A^2, symmetric), 2 m^2 n (B X)."""
    syrk = poly = apply_ = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        syrk += m * m * n
        poly += m ** 3
        apply_ += 2 * m * m * n
    return {"ns_syrk": syrk * iters, "ns_poly": poly * iters, "ns_apply": apply_ * iters}


def hbm_bytes(shapes, grad_bytes, compute_bytes, momentum=True):
    """Algorithmic HBM bytes per step of the streaming kernels.
    momentum_prep (one or more NS iterations): read G and M, write M and the operand X
    in the compute dtype (or read x, write X); momentum_sumsq (the iters == 0 path):
    read G and M, write M (or read x only).  The scaled operand rewrite (prep_operand)
    only runs for norms outside the deferral range, so it has no per-step bytes."""
    numel = sum(r * c for r, c in shapes)
    mom = numel * (grad_bytes + 8) if momentum else numel * grad_bytes
    return {"momentum_prep": mom + numel * compute_bytes, "momentum_sumsq": mom}


def measure_sign_tail(mo, torch, dev, numel, workers=8, reps=20):
    """HBM roofline of the Sign-Muon kernels at a size where bandwidth, not launch
    latency, decides: sign_pack reads 4 B and writes 1/8 B per element (fp32 input);
    sign_vote reads workers/8 B and writes 1/8 B per element; sign_unpack reads 1/8 B
    and writes 2 B (bf16 out); sign_apply reads 1/8 B and reads and writes 4 B (fp32
    weight)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    u = torch.randn(numel, generator=gen, device=dev, dtype=torch.float32)
    nwords = (numel + 31) // 32
    packed = torch.empty((workers, nwords), dtype=torch.int32, device=dev)
    out = torch.empty(nwords, dtype=torch.int32, device=dev)
    for i in range(workers):
        mo.sign_pack(u, packed[i])
    mo.sign_vote(packed, numel, out_packed=out)
    torch.cuda.synchronize()
    signs = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    weight = torch.zeros(numel, dtype=torch.float32, device=dev)
    mo.sign_unpack(out, numel, out=signs)
    mo.sign_apply(out, weight, 1e-3)
    torch.cuda.synchronize()
    mo.profile_begin()
    for _ in range(reps):
        mo.sign_pack(u, packed[0])
        mo.sign_vote(packed, numel, out_packed=out)
        mo.sign_unpack(out, numel, out=signs)
        mo.sign_apply(out, weight, 1e-3)
    torch.cuda.synchronize()
    k = mo.profile_end()
    bytes_per = {"sign_pack": numel * (4 + 1 / 8), "sign_vote": numel * (workers + 1) / 8,
                 "sign_unpack": numel * (1 / 8 + 2), "sign_apply": numel * (1 / 8 + 8)}
    res = {"numel": numel, "workers": workers}
    for name, nb in bytes_per.items():
        t = k[name][1] / k[name][0]
        res[name] = {"ms": round(t, 4), "gbs": round(nb / t / 1e6, 1),
                     "frac_hbm": round(nb / t / 1e6 / PEAK_HBM_GBS, 4)}
    del u, packed, out, signs, weight
    return res


def traffic_of(kind, workload):
    """HBM bytes per launch of `kind` from the committed rocprofv3 counter summary for
    this workload, or None if there is none or the library's GPU code changed since."""
    from matrix_optimizers_sharded_amd.profsummary import read_traffic, code_hash
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    val, h = read_traffic(path, kind)
    if val is None or h != code_hash():
        return None
    return val


def blas_ceiling(torch, dev, seconds=2.0):
    """What the vendor GEMM library (torch.matmul -> hipBLASLt) sustains on the NS
    product shapes on this same GPU, as a measured ceiling for the hand-written
    kernels.  Dense products, so the flop count is the full 2*m*n*k (no symmetry
    saving).  A calibration only: the library's step never calls it."""
    # (dtype, m, n, k, layout, what): "nn" multiplies row-major (m x k) by row-major
    # (k x n); "nt" multiplies row-major (m x k) by the transpose of a row-major
    # (n x k), the layout of X X^T
    cases = [("bf16", 4096, 11008, 4096, "nn", "B X at 4096 x 11008 (APPLY-like, K = 4096)"),
             ("bf16", 4096, 11008, 4096, "nt", "the same product with the second operand k-contiguous"),
             ("bf16", 4096, 4096, 11008, "nt", "X X^T at 4096 x 11008 (SYRK-like, K = 11008, dense)"),
             ("bf16", 4096, 4096, 4096, "nt", "A A^T at 4096^2 (POLY-like, dense)"),
             ("bf16", 768, 3072, 768, "nn", "B X at 768 x 3072 (K = 768)"),
             ("f32", 4096, 4096, 4096, "nt", "A A^T at 4096^2, fp32")]
    torch.backends.cuda.matmul.allow_tf32 = False
    out = []
    for dt, m, n, k, layout, what in cases:
        dtype = torch.bfloat16 if dt == "bf16" else torch.float32
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        a = torch.randn(m, k, generator=gen, device=dev).to(dtype)
        if layout == "nn":
            b = torch.randn(k, n, generator=gen, device=dev).to(dtype)
        else:
            b = torch.randn(n, k, generator=gen, device=dev).to(dtype).t()
        c = torch.empty(m, n, device=dev, dtype=dtype)
        # about a second of back-to-back products first, so the clock has settled
        # where a long GEMM-bound step runs, then about two seconds timed
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        est = max(time.perf_counter() - t0, 1e-5)
        for _ in range(int(1.0 / est) + 1):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        reps = max(int(seconds / est), 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * m * n * k / (ms / 1e3) / 1e12
        peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_TFLOPS
        out.append({"dtype": dt, "m": m, "n": n, "k": k, "layout": layout, "what": what, "ms": round(ms, 4),
                    "reps": reps, "tflops": round(tf, 1), "frac": round(tf / peak, 4)})
        print(f"[bench] torch.matmul {what}: {ms:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / peak:.1f}%)",
              file=sys.stderr, flush=True)
        del a, b, c
    return out


def copy_ceiling(torch, dev, nbytes=4 << 30, reps=20):
    """What a plain device-to-device copy (torch's copy kernel) moves on this GPU, read
    plus write bytes per second: the practical ceiling for the streaming kernels,
    which read and write in a similar mix."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * nbytes / (ms / 1e3) / 1e9
    print(f"[bench] device copy of {nbytes >> 20} MiB: {ms:.3f} ms, {gbs:.0f} GB/s read+write", file=sys.stderr,
          flush=True)
    del src, dst
    return {"bytes": nbytes, "ms": round(ms, 4), "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}


def cpu_info():
    """CPU model, logical core count and the BLAS library numpy calls (name, version,
    threads) on this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = {"name": p.get("internal_api"), "version": p.get("version"),
                        "threads": p.get("num_threads")}
                break
    except Exception:
        pass
    return {"cpu_model": model, "logical_cores": os.cpu_count(), "blas": blas}


def cpu_baseline(wid, iters):
    """The fp64 oracle (numpy + the host BLAS), on the host cores, as a baseline.

    Every distinct NS shape of the workload is timed once on its first matrix (a
    tall matrix counts with its transpose: the oracle works on the wide
    orientation); the whole owner set's time is the sum of those times weighted by
    how many matrices share each shape, so the figure is extrapolated unless every
    matrix was timed (the single-matrix workload)."""
    import oracle
    from matrix_optimizers_sharded_amd.workloads import WORKLOADS, host_matrix, MUON_ABC, BETA, EPS
    w = WORKLOADS[wid]
    shapes = w.shapes
    groups = {}
    for i, s in enumerate(shapes):
        groups.setdefault((min(s), max(s)), []).append(i)
    total_s, timed, parts = 0.0, 0, []
    for key, idx in groups.items():
        d = host_matrix(wid, idx[0])
        t0 = time.perf_counter()
        if wid == 5:
            oracle.ns_orthogonalize(d["mom"], *MUON_ABC, iters, EPS)
        else:
            oracle.muon_step(d["grad"], d["mom"], BETA, *MUON_ABC, iters, EPS)
        dt = time.perf_counter() - t0
        total_s += dt * len(idx)
        timed += 1
        parts.append(f"{shapes[idx[0]][0]}x{shapes[idx[0]][1]} {dt:.2f} s x {len(idx)}")
    info = cpu_info()
    threads = (info["blas"] or {}).get("threads") or info["logical_cores"]
    return {"value": w.numel / total_s, "unit": "matrix params/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": timed < w.count, "owner_set_seconds": round(total_s, 2),
            "sample": f"fp64 numpy oracle, {'NS' if wid == 5 else 'momentum + NS'}({iters}): one matrix of each "
                      f"distinct shape timed ({'; '.join(parts)}), weighted by how many matrices of the "
                      f"{w.name} set have that shape",
            **info}


class Run:
    """One workload resident on the device, with the step the benchmark times."""

    def __init__(self, mo, torch, dev, wid, compute, apply=False):
        from matrix_optimizers_sharded_amd.workloads import WORKLOADS, device_matrix, MUON_ABC, BETA, EPS
        w = WORKLOADS[wid]
        self.w, self.wid, self.compute = w, wid, compute
        shapes = w.shapes
        ws = mo.Workspace(dev)
        self.ws = ws
        if wid == 5:
            moms = [device_matrix(5, i, dev)[1] for i in range(w.count)]
            # the workers' directions side by side, so one launch packs them all
            stack = torch.empty((w.count,) + tuple(shapes[0]), dtype=torch.bfloat16, device=dev)
            outs = [stack[i] for i in range(w.count)]
            numel = shapes[0][0] * shapes[0][1]
            nwords = (numel + 31) // 32
            packed = torch.empty((w.count, nwords), dtype=torch.int32, device=dev)
            vote = torch.empty(nwords, dtype=torch.int32, device=dev)
            self.tensors = [moms, stack, packed, vote]

            def step():
                mo.ns_orthogonalize(moms, outs, *MUON_ABC, w.iters, EPS, compute=compute, workspace=ws)
                mo.sign_pack_batched(stack.view(w.count, numel), packed)
                mo.sign_vote(packed, numel, out_packed=vote)
        else:
            grads, moms = [], []
            for i in range(w.count):
                g, m = device_matrix(wid, i, dev)
                grads.append(g)
                moms.append(m)
            out_dtype = torch.bfloat16 if compute == torch.bfloat16 else torch.float32
            if apply:
                # weights: small values, updated in place every step
                outs = [(torch.randn(s, device=dev) * 0.02).to(out_dtype) for s in shapes]

                def step():
                    mo.muon_step_apply(grads, moms, outs, BETA, *MUON_ABC, w.iters, 1e-3, EPS, compute=compute,
                                       workspace=ws)
            else:
                outs = [torch.empty(s, dtype=out_dtype, device=dev) for s in shapes]

                def step():
                    mo.muon_step_batched(grads, moms, outs, BETA, *MUON_ABC, w.iters, EPS, compute=compute,
                                         workspace=ws)
            self.tensors = [grads, moms, outs]
        self.step = step
        torch.cuda.synchronize()

    def time(self, mo, torch, steps, warmup, log=True):
        """warmup untimed steps, then `steps` steps back to back between two device
        synchronisations; per-kernel times from the library's HIP events."""
        for i in range(warmup):
            self.step()
            torch.cuda.synchronize()
            if log:
                print(f"[bench] {self.w.name}: warmup {i + 1}/{warmup} done", file=sys.stderr, flush=True)
        mo.profile_begin()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kernels = mo.profile_end()
        return (t1 - t0) * 1000.0 / steps, kernels

    def release(self, torch):
        self.tensors = None
        self.ws.buf = None
        self.step = None
        torch.cuda.empty_cache()


def summarize(w, compute_bf16, ms, kernels, steps):
    """TFLOP/s, % of the dtype's MFMA peak and a per-kernel breakdown for one timed
    workload; returns (summary dict, per-launch helper)."""
    shapes = w.shapes
    flops = ns_flops(shapes, w.iters)
    f_alg = sum(flops.values())
    tflops = f_alg / (ms / 1000.0) / 1e12
    peak = PEAK_BF16_TFLOPS if compute_bf16 else PEAK_F32_TFLOPS
    es = 2 if compute_bf16 else 4
    gb = 2 if w.grad_dtype == "bf16" else 4
    hbm = hbm_bytes(shapes, 4 if w.wid == 5 else gb, es, momentum=(w.wid != 5))
    if w.wid == 5:
        one = shapes[0][0] * shapes[0][1]
        hbm["sign_pack"] = w.count * one * (es + 1 / 8)
        hbm["sign_vote"] = one * (w.count + 1) / 8

    def per_launch(name):
        launches, total = kernels[name][:2]
        lps = launches / steps
        work = flops.get(name, hbm.get(name, 0.0)) / lps
        return lps, total / launches, work

    breakdown = {}
    for name in kernels:
        lps, pl_ms, work = per_launch(name)
        entry = {"launches_per_step": lps, "ms_per_launch": round(pl_ms, 4), "ms_per_step": round(pl_ms * lps, 4)}
        if name in flops and lps > w.iters + 0.5:
            # the library ran this product as two halves on two streams at once: its
            # flops over the time at least one half was running (the union of their
            # intervals) is a lower bound on its rate, since in that time the other
            # products' halves ran beside it too
            busy = kernels[name][2] / steps
            entry.update({"two_streams": True, "busy_ms_per_step": round(busy, 4),
                          "tflops_lower_bound": round(flops[name] / (busy / 1e3) / 1e12, 2)})
        elif name in flops:
            entry["tflops"] = round(work / (pl_ms / 1e3) / 1e12, 2)
        elif name in hbm:
            entry["gbs"] = round(work / (pl_ms / 1e3) / 1e9, 1)
        breakdown[name] = entry
    out = {"ms_per_step": round(ms, 4), "params_per_s": w.numel / (ms / 1000.0), "tflops": round(tflops, 2),
           "peak_tflops": peak, "frac": round(tflops / peak, 4), "flops_per_step": f_alg, "kernels": breakdown}
    return out, per_launch, flops, hbm, peak


# The owner sets timed besides the headline one (name, compute, steps, warmup):
# every configuration of the benchmark, and the fp32 path on a multi-tile set.
OTHER = [("125m-class", "bf16", 20, 3), ("1b-class-swiglu", "bf16", 10, 2), ("sign-vote-8x4096", "bf16", 10, 2),
         ("single-256x128", "f32", 50, 5), ("1b-class-swiglu", "f32", 3, 1)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="7b-class", choices=sorted(NAMES))
    ap.add_argument("--compute", default=None, choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the named workload (by default the other owner sets follow it)")
    ap.add_argument("--sign-tail-numel", type=int, default=None,
                    help="also time sign_pack (fp32 input) and an 8-worker sign_vote on this many elements "
                         "(default: 2^28 for the sign-vote workload, off otherwise)")
    ap.add_argument("--apply", action="store_true",
                    help="time muon_step_apply (W <- W - lr*U fused into the last product, bf16 weights) "
                         "instead of muon_step_batched")
    ap.add_argument("--blas-ceiling", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the NS product shapes: a measured ceiling")
    ap.add_argument("--blas-only", action="store_true",
                    help="only the torch.matmul ceiling (for profiling the vendor kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the owner-local step needs "
              "no collective, so each GPU runs its own owner set and one GPU's rate is measured here.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_optimizers_sharded_amd as mo
    from matrix_optimizers_sharded_amd.workloads import WORKLOADS, MUON_ABC, BETA

    dev = torch.device("cuda:0")
    if args.blas_only:
        print(json.dumps({"blas_ceiling": blas_ceiling(torch, dev), "copy_ceiling": copy_ceiling(torch, dev)}),
              flush=True)
        return

    wid = NAMES[args.workload]
    w = WORKLOADS[wid]
    mo.load_library()
    compute_name = args.compute or w.compute
    compute = torch.bfloat16 if compute_name == "bf16" else torch.float32
    print(f"[bench] workload {w.name}: {w.count} matrices, {w.numel / 1e9:.3f} G params, compute {compute_name}",
          file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] 1 GiB calibration copy done", file=sys.stderr, flush=True)

    run = Run(mo, torch, dev, wid, compute, apply=args.apply)
    print("[bench] inputs resident", file=sys.stderr, flush=True)
    ms, kernels = run.time(mo, torch, args.steps, args.warmup)
    run.release(torch)
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    summary, per_launch, flops, hbm, peak = summarize(w, compute == torch.bfloat16, ms, kernels, args.steps)
    # the kernel kind that occupies the step longest (busy time: overlapping halves once)
    dom = max(kernels.items(), key=lambda kv: kv[1][2])[0] if kernels else None
    roofline = None
    if dom in flops:
        _, pl_ms, work = per_launch(dom)
        achieved = work / (pl_ms / 1e3) / 1e12
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic_of(dom, w.name)}
        if summary["kernels"][dom].get("two_streams"):
            # two half launches ran at once, beside the other products' halves: a lower
            # bound (see tflops_lower_bound); the counters were taken per half launch
            achieved = summary["kernels"][dom]["tflops_lower_bound"]
            roofline.update({"achieved": achieved, "frac": round(achieved / peak, 4), "traffic": None,
                             "two_streams": True, "lower_bound": True})
    elif dom in hbm:
        _, pl_ms, work = per_launch(dom)
        achieved = work / (pl_ms / 1e3) / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_of(dom, w.name)}

    sign_tail = None
    tail_numel = args.sign_tail_numel if args.sign_tail_numel is not None else (1 << 28 if wid == 5 else 0)
    if tail_numel:
        sign_tail = measure_sign_tail(mo, torch, dev, tail_numel)

    others = None
    if not args.no_other_workloads:
        others = []
        for name, cname, steps, warmup in OTHER:
            if name == w.name and cname == compute_name:
                continue
            ow = WORKLOADS[NAMES[name]]
            oc = torch.bfloat16 if cname == "bf16" else torch.float32
            r = Run(mo, torch, dev, ow.wid, oc)
            oms, ok = r.time(mo, torch, steps, warmup, log=False)
            r.release(torch)
            osum = summarize(ow, oc == torch.bfloat16, oms, ok, steps)[0]
            osum["kernels"] = {k: {kk: v[kk] for kk in ("ms_per_launch", "ms_per_step", "tflops", "gbs", "two_streams",
                                                     "busy_ms_per_step", "tflops_lower_bound") if kk in v}
                               for k, v in osum["kernels"].items()}
            print(f"[bench] {name} ({cname}): {oms:.3f} ms/step, {osum['tflops']} TFLOP/s ({100 * osum['frac']:.1f}% "
                  f"of {osum['peak_tflops']})", file=sys.stderr, flush=True)
            others.append({"workload": name, "dtype": cname, "steps": steps, "warmup": warmup, **osum})

    ceiling = {"gemm": blas_ceiling(torch, dev), "copy": copy_ceiling(torch, dev)} if args.blas_ceiling else None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wid, w.iters)

    line = {
        "metric": "NS-orthogonalized params/sec + MFMA TFLOP/s (% peak), 7B layer shapes",
        "value": w.numel / (ms / 1000.0),
        "unit": "matrix params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_name,
        "data": "synthetic",
        "config": {"workload": w.name, "matrices": w.count, "params": w.numel, "ns_iters": w.iters,
                   "grad_dtype": w.grad_dtype, "momentum_dtype": "f32", "accumulate": "f32",
                   "coefficients": list(MUON_ABC), "beta": BETA, "parallelism": "single GPU (owner-local)",
                   "step": "muon_step_apply (W -= lr*U fused)" if args.apply else "muon_step_batched"},
        "tflops": summary["tflops"],
        "pct_peak": round(100.0 * summary["frac"], 2),
        "flops_per_step": summary["flops_per_step"],
        "kernels": summary["kernels"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sign_tail": sign_tail,
        "other_workloads": others,
    }
    if ceiling is not None:
        line["blas_ceiling"] = ceiling
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
