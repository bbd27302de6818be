"""GPU parity where every GEMM launch holds more tiles than its persistent grid has
blocks, so each block walks several tiles: the cross-tile operand ring, the
next-tile setup and (fp32) the eight-loader slab layout all run.  The owner steps
every whole matrix it holds ("Riassunto Tecnico: MatrixFSDP", Metodologia item 1),
so a batch of many matrices is the ordinary case.

The whole 72-matrix 125M-class owner set is the workload: 432 SYRK/POLY tiles and
1296 APPLY tiles per launch against a grid of at most 256 blocks.  Bars: fp32
compute <= 1e-4, bf16 compute <= 2e-2 relative Frobenius error per matrix, momentum
state bit-exact for every matrix."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import MUON_ABC, BETA, EPS, WORKLOADS, host_matrix, f32_to_bf16_bits
from gpu_util import say, to_dev_f32, to_dev_bf16, host_f32, rel_err, gaussian, bf16_round

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TILE = 256
# checked against the oracle one by one: each shape from the first and the last layer
SAMPLE = [0, 3, 4, 5, 66, 69, 70, 71]


def tile_counts(shapes):
    """(SYRK/POLY tiles, APPLY tiles) of one launch over the owner set: upper 256x256
    tiles of the m x m Gram matrix, all tiles of the m x n operand."""
    tri = rect = 0
    for r, c in shapes:
        tm = -(-min(r, c) // TILE)
        tn = -(-max(r, c) // TILE)
        tri += tm * (tm + 1) // 2
        rect += tm * tn
    return tri, rect


def max_grid():
    """The persistent GEMM grid: one block per CU, rounded down to a multiple of 8."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return cus // 8 * 8 if cus >= 8 else cus


def _inputs():
    ins = [host_matrix(2, i) for i in range(WORKLOADS[2].count)]
    return ins


def _assert_multitile(shapes):
    tri, rect = tile_counts(shapes)
    g = max_grid()
    say(f"tiles per launch: SYRK/POLY {tri}, APPLY {rect}; grid {g}")
    assert tri > g and rect > g, (tri, rect, g)


@pytest.mark.parametrize("grad_dtype", ["bf16", "f32"])
def test_125m_class_fp32_compute_multitile(gpu, grad_dtype):
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched
    w = WORKLOADS[2]
    _assert_multitile(w.shapes)
    ins = _inputs()
    say(f"125m-class, 72 matrices, fp32 compute, {grad_dtype} grads")
    if grad_dtype == "bf16":
        grads_np = [d["grad"] for d in ins]
        grads = [to_dev_bf16(d["grad_bits"], gpu) for d in ins]
    else:
        # fp32 gradients that are not bf16-representable: add a small fp32 offset
        grads_np = [(d["grad"] + gaussian(d["shape"], 900 + i, 1e-4)).astype(np.float32) for i, d in enumerate(ins)]
        grads = [to_dev_f32(g, gpu) for g in grads_np]
    moms = [to_dev_f32(d["mom"], gpu) for d in ins]
    outs = [torch.empty(d["shape"], dtype=torch.float32, device=gpu) for d in ins]
    muon_step_batched(grads, moms, outs, BETA, *MUON_ABC, w.iters, EPS, compute=torch.float32)
    torch.cuda.synchronize()
    for i, d in enumerate(ins):
        want_m = oracle.momentum_state_fp32(grads_np[i], d["mom"], BETA)
        np.testing.assert_array_equal(host_f32(moms[i]).view(np.uint32), want_m.view(np.uint32),
                                      err_msg=f"matrix {i}: momentum state")
    worst = 0.0
    for i in SAMPLE:
        _, want_u = oracle.muon_step(grads_np[i], ins[i]["mom"], BETA, *MUON_ABC, w.iters, EPS)
        e = rel_err(host_f32(outs[i]), want_u)
        worst = max(worst, e)
        assert e <= TOL["f32"], f"matrix {i} {ins[i]['shape']}: rel err {e:.3e}"
    say(f"  worst rel err over the sample {worst:.3e}")


def test_125m_class_bf16_compute_f32_out_multitile(gpu):
    """The bf16 path writing fp32 U, the whole set: every matrix checked."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched
    w = WORKLOADS[2]
    _assert_multitile(w.shapes)
    ins = _inputs()
    grads = [to_dev_bf16(d["grad_bits"], gpu) for d in ins]
    moms = [to_dev_f32(d["mom"], gpu) for d in ins]
    outs = [torch.empty(d["shape"], dtype=torch.float32, device=gpu) for d in ins]
    muon_step_batched(grads, moms, outs, BETA, *MUON_ABC, w.iters, EPS, compute=torch.bfloat16)
    torch.cuda.synchronize()
    worst = 0.0
    for i, d in enumerate(ins):
        want_m, want_u = oracle.muon_step(d["grad"], d["mom"], BETA, *MUON_ABC, w.iters, EPS)
        np.testing.assert_array_equal(host_f32(moms[i]).view(np.uint32), want_m.view(np.uint32))
        e = rel_err(host_f32(outs[i]), want_u)
        worst = max(worst, e)
        assert e <= TOL["bf16"], f"matrix {i} {d['shape']}: rel err {e:.3e}"
    say(f"  worst rel err over all 72 matrices {worst:.3e}")


@pytest.mark.parametrize("compute,wdt", [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")])
def test_125m_class_step_apply_multitile(gpu, compute, wdt):
    """muon_step_apply over the whole set: W <- W - lr*U fused into the last product.
    fp32 weights: (W_old - W_new)/lr is U within the path's bar.  bf16 weights: each
    element is within half a bf16 ulp of the exact update plus the direction's
    error."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_apply
    w = WORKLOADS[2]
    _assert_multitile(w.shapes)
    ins = _inputs()
    lr = 0.25 if wdt == "f32" else 0.05
    say(f"125m-class muon_step_apply compute={compute} weights={wdt}")
    grads = [to_dev_bf16(d["grad_bits"], gpu) for d in ins]
    moms = [to_dev_f32(d["mom"], gpu) for d in ins]
    w0 = []
    for i, d in enumerate(ins):
        x = gaussian(d["shape"], 1300 + i, 0.02 if wdt == "f32" else 0.5)
        w0.append(bf16_round(x)[1] if wdt == "bf16" else x)
    if wdt == "bf16":
        wts = [to_dev_bf16(f32_to_bf16_bits(x), gpu) for x in w0]
    else:
        wts = [to_dev_f32(x, gpu) for x in w0]
    muon_step_apply(grads, moms, wts, BETA, *MUON_ABC, w.iters, lr, EPS, compute=tdt(compute))
    torch.cuda.synchronize()
    lr32 = float(np.float32(lr))
    worst = 0.0
    for i in SAMPLE:
        d = ins[i]
        want_m, u = oracle.muon_step(d["grad"], d["mom"], BETA, *MUON_ABC, w.iters, EPS)
        np.testing.assert_array_equal(host_f32(moms[i]).view(np.uint32), want_m.view(np.uint32))
        got = host_f32(wts[i]).astype(np.float64)
        if wdt == "f32":
            e = rel_err((w0[i].astype(np.float64) - got) / lr32, u)
            worst = max(worst, e)
            assert e <= TOL[compute], (i, d["shape"], e)
        else:
            want = oracle.weight_update(w0[i], u, lr)
            half_ulp = np.abs(want) * 2.0 ** -8 + 1e-30
            resid = np.maximum(np.abs(got - want) - half_ulp, 0.0)
            bound = lr32 * TOL["bf16"] * np.linalg.norm(u)
            assert np.linalg.norm(resid) <= bound + 1e-12, (i, d["shape"], float(np.linalg.norm(resid)))
    say(f"  worst direction rel err {worst:.3e}")


def tdt(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]
