"""The allocation-free entry point, muon_step_batched_noalloc, through the C ABI:
on the same inputs its results equal muon_step_batched's bit for bit (the same
kernels in the same order; only the scratch address differs), and both stay
within the oracle's bar.  Two calls in a row on the one per-GPU scratch, the second
on a smaller list, so leftovers of the first call must not leak into the second."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import MUON_ABC, BETA, EPS, f32_to_bf16_bits
from gpu_util import say, to_dev_f32, to_dev_bf16, host_f32, rel_err, gaussian, bf16_round

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _inputs(shapes, seed, std=0.02):
    grads = [bf16_round(gaussian(s, seed + i, std))[1] for i, s in enumerate(shapes)]
    moms = [gaussian(s, seed + 100 + i, std) for i, s in enumerate(shapes)]
    return grads, moms


def _run(gpu, fn, grads, moms, compute, out_dtype, **kw):
    import torch
    g = [to_dev_bf16(f32_to_bf16_bits(x), gpu) for x in grads]
    m = [to_dev_f32(x, gpu) for x in moms]
    o = [torch.empty(x.shape, dtype=out_dtype, device=gpu) for x in grads]
    torch.cuda.synchronize()
    fn(g, m, o, BETA, *MUON_ABC, 5, EPS, compute=compute, **kw)
    torch.cuda.synchronize()
    return [host_f32(x) for x in m], [host_f32(x) for x in o]


def _compare(gpu, shapes, seed, compute_name):
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched, muon_step_batched_noalloc, workspace_bytes
    compute = torch.float32 if compute_name == "f32" else torch.bfloat16
    out_dtype = torch.float32 if compute_name == "f32" else torch.bfloat16
    need = workspace_bytes(shapes, compute)
    say(f"noalloc {compute_name} shapes {shapes}: {need / 2**20:.1f} MiB of scratch")
    grads, moms = _inputs(shapes, seed)
    m_na, u_na = _run(gpu, muon_step_batched_noalloc, grads, moms, compute, out_dtype)
    m_ws, u_ws = _run(gpu, muon_step_batched, grads, moms, compute, out_dtype)
    for i, s in enumerate(shapes):
        np.testing.assert_array_equal(m_na[i].view(np.uint32), m_ws[i].view(np.uint32), err_msg=f"{s} momentum")
        np.testing.assert_array_equal(u_na[i].view(np.uint32), u_ws[i].view(np.uint32), err_msg=f"{s} U")
        want_m, want_u = oracle.muon_step(grads[i], moms[i], BETA, *MUON_ABC, 5, EPS)
        np.testing.assert_array_equal(m_na[i].view(np.uint32), want_m.view(np.uint32))
        e = rel_err(u_na[i], want_u)
        assert e <= TOL[compute_name], (s, e)


@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(gpu, compute):
    # first call: several tiles per launch, ragged and transposed shapes
    _compare(gpu, [(768, 3072), (3072, 768), (768, 768), (300, 520), (520, 300)], 10, compute)
    # second call on the same scratch: a smaller list
    _compare(gpu, [(257, 129), (200, 600)], 20, compute)


def test_noalloc_rejects_lists_beyond_its_scratch(gpu):
    import torch
    from matrix_optimizers_sharded_amd import (MatoptError, muon_step_batched_noalloc, workspace_bytes,
                                               NOALLOC_SCRATCH_BYTES)
    shapes = [(4096, 4096), (4096, 4096)]
    assert workspace_bytes(shapes, torch.bfloat16) > NOALLOC_SCRATCH_BYTES
    g = [torch.zeros(s, dtype=torch.bfloat16, device=gpu) for s in shapes]
    m = [torch.zeros(s, dtype=torch.float32, device=gpu) for s in shapes]
    o = [torch.empty(s, dtype=torch.bfloat16, device=gpu) for s in shapes]
    with pytest.raises(MatoptError) as ei:
        muon_step_batched_noalloc(g, m, o, BETA, *MUON_ABC, 5, EPS)
    assert ei.value.code == -3
    torch.cuda.synchronize()
    # the step still works afterwards
    _compare(gpu, [(256, 128)], 30, "f32")
