"""GPU parity for the rows after the hot path: the fused weight update
(muon_step_apply), the Sign-Muon weight update from the voted bits (sign_apply) and
the unpack for the local polar step on the voted signs (sign_unpack), through the C
ABI against the fp64 oracle.  Bars: integer and bit-level stages bit-exact; the NS
direction within the path's bars (fp32 compute 1e-4, bf16 compute 2e-2 relative
Frobenius error)."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import MUON_ABC, BETA, EPS, f32_to_bf16_bits
from gpu_util import say, to_dev_f32, to_dev_bf16, host_f32, rel_err, gaussian, bf16_round

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def tdt(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def random_words(numel, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 2 ** 32, (numel + 31) // 32, dtype=np.uint64).astype(np.uint32)
    if numel % 32:
        w[-1] &= np.uint32((1 << (numel % 32)) - 1)
    return w


def dev_words(words, dev):
    import torch
    return torch.from_numpy(words.view(np.int32).copy()).to(dev)


# ---------------------------------------------------------------- sign_unpack

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 7, 8, 31, 33, 100, 4099, 65536 + 13])
def test_sign_unpack_bit_exact(gpu, dtype, numel):
    import torch
    from matrix_optimizers_sharded_amd import sign_unpack
    say(f"sign_unpack dtype={dtype} numel={numel}")
    words = random_words(numel, numel)
    out = sign_unpack(dev_words(words, gpu), numel, dtype=tdt(dtype))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_f32(out), oracle.unpack_signs(words, numel))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sign_unpack_unaligned_output(gpu, dtype):
    import torch
    from matrix_optimizers_sharded_amd import sign_unpack
    numel = 1000
    words = random_words(numel, 5)
    buf = torch.zeros(numel + 1, dtype=tdt(dtype), device=gpu)
    sign_unpack(dev_words(words, gpu), numel, out=buf[1:])          # one element off: scalar path
    torch.cuda.synchronize()
    got = host_f32(buf)
    assert got[0] == 0.0
    np.testing.assert_array_equal(got[1:], oracle.unpack_signs(words, numel))


# ---------------------------------------------------------------- sign_apply

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 9, 32, 33, 1000, 65536 + 5])
@pytest.mark.parametrize("lr", [1e-3, -0.3])
def test_sign_apply_bit_exact(gpu, dtype, numel, lr):
    import torch
    from matrix_optimizers_sharded_amd import sign_apply
    say(f"sign_apply dtype={dtype} numel={numel} lr={lr}")
    words = random_words(numel, 3 * numel + 1)
    w0 = gaussian(numel, numel, 0.02)
    if dtype == "bf16":
        bits, w0 = bf16_round(w0)
        w = to_dev_bf16(bits, gpu)
    else:
        w = to_dev_f32(w0, gpu)
    sign_apply(dev_words(words, gpu), w, lr)
    torch.cuda.synchronize()
    want = oracle.sign_update(w0, words, lr, bf16=(dtype == "bf16"))
    np.testing.assert_array_equal(host_f32(w).astype(np.float64), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sign_apply_unaligned_weight(gpu, dtype):
    """A weight view one element past a 16-byte boundary takes the element-by-element
    path; the element before the view is left alone."""
    import torch
    from matrix_optimizers_sharded_amd import sign_apply
    numel = 5000
    say(f"sign_apply unaligned dtype={dtype} numel={numel}")
    words = random_words(numel, 11)
    w0 = gaussian(numel + 1, 12, 0.02)
    if dtype == "bf16":
        bits, w0 = bf16_round(w0)
        buf = to_dev_bf16(bits, gpu)
    else:
        buf = to_dev_f32(w0, gpu)
    sign_apply(dev_words(words, gpu), buf[1:], 1e-3)
    torch.cuda.synchronize()
    got = host_f32(buf).astype(np.float64)
    assert got[0] == w0[0]
    np.testing.assert_array_equal(got[1:], oracle.sign_update(w0[1:], words, 1e-3, bf16=(dtype == "bf16")))


def test_vote_then_apply_and_polar_step(gpu):
    """Sign-Muon's distributed flow on one GPU: pack 5 workers' directions, vote,
    update the weight with the voted signs (item 4), and the optional local polar
    step on the voted sign matrix (item 5: unpack, then ns_orthogonalize)."""
    import torch
    from matrix_optimizers_sharded_amd import sign_pack, sign_vote, sign_unpack, sign_apply, ns_orthogonalize
    rows, cols, M = 300, 520, 5
    us = [gaussian((rows, cols), 40 + k) for k in range(M)]
    numel = rows * cols
    nwords = (numel + 31) // 32
    packed = torch.empty((M, nwords), dtype=torch.int32, device=gpu)
    for k in range(M):
        sign_pack(to_dev_f32(us[k], gpu), packed[k])
    voted, _ = sign_vote(packed, numel)
    w0 = gaussian((rows, cols), 99, 0.02)
    w = to_dev_f32(w0, gpu)
    sign_apply(voted, w, 0.01)
    signs = sign_unpack(voted, numel, dtype=torch.bfloat16).view(rows, cols)
    polar = torch.empty((rows, cols), dtype=torch.float32, device=gpu)
    ns_orthogonalize([signs], [polar], *MUON_ABC, 5, EPS, compute=torch.bfloat16)
    torch.cuda.synchronize()
    want_words, _ = oracle.majority_vote(np.stack([oracle.sign_pack(u) for u in us]), numel)
    np.testing.assert_array_equal(voted.cpu().numpy().view(np.uint32), want_words)
    np.testing.assert_array_equal(host_f32(w).reshape(-1).astype(np.float64),
                                  oracle.sign_update(w0, want_words, 0.01))
    s = oracle.unpack_signs(want_words, numel).reshape(rows, cols)
    err = rel_err(host_f32(polar), oracle.ns_orthogonalize(s, *MUON_ABC, 5, EPS))
    say(f"polar step on voted signs {rows}x{cols}: rel err {err:.3e}")
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------- muon_step_apply

SHAPES = [(256, 128), (1, 1), (257, 129), (129, 257), (300, 1), (512, 512), (768, 320)]


@pytest.mark.parametrize("compute", ["f32", "bf16"])
@pytest.mark.parametrize("iters", [0, 1, 5])
def test_muon_step_apply_fp32_weights(gpu, compute, iters):
    """fp32 weights: (W_old - W_new) / lr is the direction U, within the path's bar;
    the momentum state equals the exact fused multiply-add."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_apply
    say(f"muon_step_apply fp32 weights compute={compute} iters={iters}")
    lr = 0.25
    grads = [bf16_round(gaussian(s, 10 + i, 0.02))[1] for i, s in enumerate(SHAPES)]
    moms = [gaussian(s, 50 + i, 0.02) for i, s in enumerate(SHAPES)]
    w0 = [gaussian(s, 90 + i, 0.02) for i, s in enumerate(SHAPES)]
    g_dev = [to_dev_bf16(f32_to_bf16_bits(g), gpu) for g in grads]
    m_dev = [to_dev_f32(m, gpu) for m in moms]
    w_dev = [to_dev_f32(w, gpu) for w in w0]
    muon_step_apply(g_dev, m_dev, w_dev, BETA, *MUON_ABC, iters, lr, EPS, compute=tdt(compute))
    torch.cuda.synchronize()
    worst = 0.0
    for i, s in enumerate(SHAPES):
        m_state, u = oracle.muon_step(grads[i], moms[i], BETA, *MUON_ABC, iters, EPS)
        np.testing.assert_array_equal(host_f32(m_dev[i]), m_state)
        w_new = host_f32(w_dev[i]).astype(np.float64)
        direction = (w0[i].astype(np.float64) - w_new) / float(np.float32(lr))
        err = rel_err(direction, u)
        worst = max(worst, err)
        assert err <= TOL[compute], (s, err)
        # the whole update, in the oracle's terms
        want = oracle.weight_update(w0[i], u, lr)
        assert rel_err(w_new - w0[i], want - w0[i]) <= TOL[compute]
    say(f"  worst direction rel err {worst:.3e}")


@pytest.mark.parametrize("iters", [0, 5])
def test_muon_step_apply_bf16_weights(gpu, iters):
    """bf16 weights: W_new is W_old - lr*U rounded to bf16, so each element is
    within half a bf16 ulp of the exact update plus the direction's error."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_apply
    say(f"muon_step_apply bf16 weights iters={iters}")
    lr = 0.05
    for i, s in enumerate(SHAPES):
        g = bf16_round(gaussian(s, 20 + i, 0.02))[1]
        m = gaussian(s, 60 + i, 0.02)
        wb, w0 = bf16_round(gaussian(s, 95 + i, 0.5))
        m_dev = to_dev_f32(m, gpu)
        w_dev = to_dev_bf16(wb, gpu)
        muon_step_apply([to_dev_bf16(f32_to_bf16_bits(g), gpu)], [m_dev], [w_dev], BETA, *MUON_ABC, iters, lr,
                        EPS, compute=torch.bfloat16)
        torch.cuda.synchronize()
        _, u = oracle.muon_step(g, m, BETA, *MUON_ABC, iters, EPS)
        want = oracle.weight_update(w0, u, lr)
        got = host_f32(w_dev).astype(np.float64)
        half_ulp = np.abs(want) * 2.0 ** -8 + 1e-30          # bf16 has 8 significant bits
        resid = np.abs(got - want) - half_ulp
        bound = float(np.float32(lr)) * TOL["bf16"] * np.linalg.norm(u)
        assert np.linalg.norm(np.maximum(resid, 0.0)) <= bound + 1e-12, (s, float(np.linalg.norm(resid)))


def test_muon_step_apply_matches_batched_direction(gpu):
    """The fused update and muon_step_batched (fp32 out) move by the same U: the
    momentum states are bit-identical and W_old - lr*U agrees to fp32 rounding."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_apply, muon_step_batched
    shapes = [(512, 768), (768, 512), (300, 300)]
    grads = [gaussian(s, 7 + i, 0.02) for i, s in enumerate(shapes)]
    moms = [gaussian(s, 17 + i, 0.02) for i, s in enumerate(shapes)]
    w0 = [gaussian(s, 27 + i, 0.02) for i, s in enumerate(shapes)]
    lr = 0.125
    m_a = [to_dev_f32(m, gpu) for m in moms]
    m_b = [to_dev_f32(m, gpu) for m in moms]
    w = [to_dev_f32(x, gpu) for x in w0]
    outs = [torch.empty(s, dtype=torch.float32, device=gpu) for s in shapes]
    muon_step_apply([to_dev_f32(g, gpu) for g in grads], m_a, w, BETA, *MUON_ABC, 5, lr, EPS,
                    compute=torch.bfloat16)
    muon_step_batched([to_dev_f32(g, gpu) for g in grads], m_b, outs, BETA, *MUON_ABC, 5, EPS,
                      compute=torch.bfloat16)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        np.testing.assert_array_equal(host_f32(m_a[i]), host_f32(m_b[i]))
        want = w0[i].astype(np.float64) - float(np.float32(lr)) * host_f32(outs[i]).astype(np.float64)
        got = host_f32(w[i]).astype(np.float64)
        assert np.max(np.abs(got - want)) <= 2.0 ** -22 * np.max(np.abs(want)), i
