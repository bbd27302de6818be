"""A step captured in a HIP graph (torch.cuda.graph) and replayed: every replay must
equal an eager call on the same inputs, bit for bit.  The library records no
memsets or copies (the descriptor table travels in kernel arguments, which the
graph keeps by value), and under capture it keeps every product on the capturing
stream.  Replays are separated by eager work and synchronisations, and the inputs
are reset before each one, since the step updates the momentum in place."""

import numpy as np
import pytest

from matrix_optimizers_sharded_amd.workloads import MUON_ABC, BETA, EPS, f32_to_bf16_bits
from gpu_util import say, to_dev_f32, to_dev_bf16, host_f32, gaussian, bf16_round

pytestmark = pytest.mark.gpu

# both product paths (m > 256 on 256-tiles, m <= 256 on 32-blocks) and more than
# one matrix, which outside capture would take the two-stream split
SHAPES = [(768, 768), (512, 1024), (1024, 512), (300, 200)]


def _inputs(gpu):
    grads = [bf16_round(gaussian(s, 1200 + i, 0.02))[1] for i, s in enumerate(SHAPES)]
    moms = [gaussian(s, 1300 + i, 0.02) for i, s in enumerate(SHAPES)]
    g_dev = [to_dev_bf16(f32_to_bf16_bits(g), gpu) for g in grads]
    m0 = [to_dev_f32(m, gpu) for m in moms]
    return g_dev, m0


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_captured_step_replays_equal_the_eager_call(gpu, entry):
    import torch
    import matrix_optimizers_sharded_amd as mo
    say(f"graph capture of the step ({entry}), 3 replays")
    g_dev, m0 = _inputs(gpu)
    m_dev = [m.clone() for m in m0]
    outs = [torch.empty(s, dtype=torch.bfloat16, device=gpu) for s in SHAPES]
    ws = mo.Workspace(gpu)

    def step():
        if entry == "noalloc":
            mo.muon_step_batched_noalloc(g_dev, m_dev, outs, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16)
        else:
            mo.muon_step_batched(g_dev, m_dev, outs, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16,
                                 workspace=ws)

    # eager reference (this call also sizes the workspace, so capture allocates nothing)
    step()
    torch.cuda.synchronize()
    ref_u = [host_f32(o) for o in outs]
    ref_m = [host_f32(m) for m in m_dev]

    graph = torch.cuda.CUDAGraph()
    for m, m_init in zip(m_dev, m0):
        m.copy_(m_init)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work between replays: reset the state, clear the outputs
        for m, m_init in zip(m_dev, m0):
            m.copy_(m_init)
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(SHAPES)):
            np.testing.assert_array_equal(host_f32(outs[i]).view(np.uint32), ref_u[i].view(np.uint32),
                                          err_msg=f"replay {r}, matrix {i}: U")
            np.testing.assert_array_equal(host_f32(m_dev[i]).view(np.uint32), ref_m[i].view(np.uint32),
                                          err_msg=f"replay {r}, matrix {i}: momentum")
    # and the eager call still works after the graph
    for m, m_init in zip(m_dev, m0):
        m.copy_(m_init)
    step()
    torch.cuda.synchronize()
    for i in range(len(SHAPES)):
        np.testing.assert_array_equal(host_f32(outs[i]).view(np.uint32), ref_u[i].view(np.uint32))
