"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by
element, on seeded inputs.  Bars: fp32 compute <= 1e-4 and bf16 compute <= 2e-2
relative Frobenius error per matrix; momentum state and all integer stages
bit-exact."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import (
    MUON_ABC, TEXTBOOK_QUINTIC_ABC, TEXTBOOK_CUBIC_ABC, BETA, EPS, WORKLOADS, host_matrix, f32_to_bf16_bits)
from gpu_util import (say, to_dev_f32, to_dev_bf16, host_f32, rel_err, gaussian, bf16_round,
                      run_muon, run_ns)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def tdt(name):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


# ---------------------------------------------------------------- sign tail

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("numel", [1, 7, 31, 32, 33, 64, 100, 1000, 4099, 65536 + 13])
def test_sign_pack_bit_exact(gpu, dtype, numel):
    import torch
    from matrix_optimizers_sharded_amd import sign_pack
    say(f"sign_pack dtype={dtype} numel={numel}")
    rng = np.random.default_rng(numel)
    v = rng.standard_normal(numel).astype(np.float32)
    v[rng.random(numel) < 0.05] = 0.0
    v[rng.random(numel) < 0.05] = -0.0
    if numel > 10:
        v[3] = np.nan
    if dtype == "bf16":
        bits, vals = bf16_round(np.nan_to_num(v, nan=0.0))
        vals = vals.copy()
        u = to_dev_bf16(bits, gpu)
    else:
        vals = v
        u = to_dev_f32(v, gpu)
    packed = sign_pack(u)
    torch.cuda.synchronize()
    got = packed.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, oracle.sign_pack(host_f32(u)))


def test_sign_pack_unaligned_view(gpu):
    import torch
    from matrix_optimizers_sharded_amd import sign_pack
    v = gaussian(1001, 3)
    u = to_dev_f32(v, gpu)[1:]          # 4-byte offset: scalar load path
    packed = sign_pack(u)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), oracle.sign_pack(v[1:]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,numel,pad", [(1, 33, 0), (3, 1, 0), (3, 31, 5), (8, 1000, 0), (8, 1000, 3),
                                         (5, 65537, 0), (2, 4096, 4)])
def test_sign_pack_batched_bit_exact(gpu, dtype, M, numel, pad):
    """One launch over M workers (rows of u, each row padded by pad values) gives
    each worker's words, bit for bit, in the [M][nwords] stack."""
    import torch
    from matrix_optimizers_sharded_amd import sign_pack_batched
    say(f"sign_pack_batched dtype={dtype} M={M} numel={numel} pad={pad}")
    rng = np.random.default_rng(M * 1000 + numel + pad)
    v = rng.standard_normal((M, numel + pad)).astype(np.float32)
    v[rng.random(v.shape) < 0.05] = 0.0
    v[rng.random(v.shape) < 0.05] = -0.0
    if dtype == "bf16":
        bits, vals = bf16_round(v)
        full = to_dev_bf16(bits, gpu)
    else:
        full = to_dev_f32(v, gpu)
    u = full[:, :numel]
    packed = sign_pack_batched(u)
    torch.cuda.synchronize()
    got = packed.cpu().numpy().view(np.uint32)
    host = host_f32(full)
    for w in range(M):
        np.testing.assert_array_equal(got[w], oracle.sign_pack(host[w, :numel]), err_msg=f"worker {w}")


@pytest.mark.parametrize("M", [1, 2, 3, 7, 8, 9, 15, 16, 127])
# 169465 elements: 5296 words, a multiple of 4: the four-word path over several
# blocks, the last one ragged
@pytest.mark.parametrize("numel", [1, 33, 1000, 65537, 169465])
def test_sign_vote_bit_exact(gpu, M, numel):
    import torch
    from matrix_optimizers_sharded_amd import sign_vote
    say(f"sign_vote M={M} numel={numel}")
    rng = np.random.default_rng(M * 7 + numel)
    packed = np.stack([oracle.sign_pack(rng.standard_normal(numel)) for _ in range(M)])
    dev = torch.from_numpy(packed.view(np.int32)).to(gpu)
    out, sums = sign_vote(dev, numel, with_sums=True)
    torch.cuda.synchronize()
    want_out, want_sums = oracle.majority_vote(packed, numel)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want_out)
    np.testing.assert_array_equal(sums.cpu().numpy().astype(np.int64), want_sums)


def test_sign_vote_large_M_without_sums(gpu):
    import torch
    from matrix_optimizers_sharded_amd import sign_vote
    M, numel = 1000, 777
    rng = np.random.default_rng(1)
    packed = rng.integers(0, 2 ** 32, size=(M, (numel + 31) // 32), dtype=np.uint64).astype(np.uint32)
    packed[:, -1] &= np.uint32((1 << (numel % 32)) - 1)
    out, _ = sign_vote(torch.from_numpy(packed.view(np.int32)).to(gpu), numel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), oracle.majority_vote(packed, numel)[0])


@pytest.mark.parametrize("M", [5, 15, 16, 255, 256, 1000])
@pytest.mark.parametrize("nwords", [1024, 3248])
def test_sign_vote_four_word_path(gpu, M, nwords):
    """nwords a multiple of 4 on a 16-byte aligned buffer takes the four-word path
    (1024 words: one block; 3248: four blocks, the last ragged); the same words on a
    base shifted by one word take the one-word path.  The M values straddle the
    counter depths (4 bit planes up to 15 workers, 8 up to 255)."""
    import torch
    from matrix_optimizers_sharded_amd import sign_vote
    numel = nwords * 32 - 3
    rng = np.random.default_rng(M)
    packed = rng.integers(0, 2 ** 32, size=(M, nwords), dtype=np.uint64).astype(np.uint32)
    packed[:, -1] &= np.uint32((1 << (numel % 32)) - 1)
    want = oracle.majority_vote(packed, numel)[0]
    dev = torch.from_numpy(packed.view(np.int32)).to(gpu)
    out, _ = sign_vote(dev, numel)
    flat = torch.zeros(M * nwords + 1, dtype=torch.int32, device=gpu)
    shifted = flat[1:].view(M, nwords)
    shifted.copy_(dev)
    out2, _ = sign_vote(shifted, numel)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want)
    np.testing.assert_array_equal(out2.cpu().numpy().view(np.uint32), want)


def test_sign_vote_two_groups_per_thread(gpu):
    """From 2^20 groups of four words on, a thread votes two groups 256 apart: here
    2^20 + 300 groups, so the last block has threads with two groups and threads with
    one.  With the int8 sums."""
    import torch
    from matrix_optimizers_sharded_amd import sign_vote
    M, nwords = 3, 4 * ((1 << 20) + 300)
    numel = nwords * 32 - 3
    say(f"sign_vote two groups per thread M={M} nwords={nwords}")
    rng = np.random.default_rng(77)
    packed = rng.integers(0, 2 ** 32, size=(M, nwords), dtype=np.uint64).astype(np.uint32)
    packed[:, -1] &= np.uint32((1 << (numel % 32)) - 1)
    out, sums = sign_vote(torch.from_numpy(packed.view(np.int32)).to(gpu), numel, with_sums=True)
    torch.cuda.synchronize()
    want_out, want_sums = oracle.majority_vote(packed, numel)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want_out)
    np.testing.assert_array_equal(sums.cpu().numpy(), want_sums.astype(np.int8))


# ---------------------------------------------------------------- Muon step

def check_muon(grads, moms, got_m, got_u, compute, abc, iters, beta=BETA, eps=EPS, label=""):
    worst = 0.0
    for i, (g, m0, gm, gu) in enumerate(zip(grads, moms, got_m, got_u)):
        want_m, want_u = oracle.muon_step(g, m0, beta, *abc, iters, eps)
        np.testing.assert_array_equal(gm.view(np.uint32), want_m.view(np.uint32),
                                      err_msg=f"{label} matrix {i}: momentum state")
        e = rel_err(gu, want_u)
        worst = max(worst, e)
        assert e <= TOL[compute], f"{label} matrix {i} shape {g.shape}: rel err {e:.3e}"
    say(f"{label}: worst rel err {worst:.3e}")
    return worst


def test_single_256x128_fp32(gpu):
    import torch
    w = WORKLOADS[1]
    inp = host_matrix(1, 0)
    say("workload single-256x128 fp32")
    gm, gu = run_muon(gpu, [inp["grad"]], [inp["mom"]], torch.float32, torch.float32, torch.float32,
                      BETA, MUON_ABC, w.iters, EPS)
    check_muon([inp["grad"]], [inp["mom"]], gm, gu, "f32", MUON_ABC, w.iters, label="single-256x128")


RAGGED = [(1, 1), (1, 300), (300, 1), (257, 129), (129, 257), (300, 200), (512, 512), (700, 260), (64, 1000)]
# Matrices with min(rows, cols) <= 256 run their products on 32 x 32 blocks, one wave
# each; larger ones on the persistent 256 x 256 tiles.  RAGGED holds both kinds.
SMALL_M = 256


@pytest.mark.parametrize("compute", ["f32", "bf16"])
@pytest.mark.parametrize("iters", [0, 1, 5])
def test_ragged_shapes(gpu, compute, iters):
    import torch
    assert any(min(s) <= SMALL_M for s in RAGGED) and any(min(s) > SMALL_M for s in RAGGED)
    say(f"ragged shapes compute={compute} iters={iters}")
    grads = [gaussian(s, 100 + i) for i, s in enumerate(RAGGED)]
    moms = [gaussian(s, 200 + i) for i, s in enumerate(RAGGED)]
    gm, gu = run_muon(gpu, grads, moms, torch.float32, tdt(compute), torch.float32, BETA, MUON_ABC, iters, EPS)
    check_muon(grads, moms, gm, gu, compute, MUON_ABC, iters, label=f"ragged {compute} k={iters}")


@pytest.mark.parametrize("compute", ["f32", "bf16"])
def test_ns_orthogonalize_and_out_dtypes(gpu, compute):
    import torch
    shapes = [(96, 320), (320, 96), (256, 256)]
    xs = [gaussian(s, 300 + i, 0.05) for i, s in enumerate(shapes)]
    for in_dt, out_dt in [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")]:
        say(f"ns_orthogonalize compute={compute} in={in_dt} out={out_dt}")
        xin = [bf16_round(x)[1] for x in xs] if in_dt == "bf16" else xs
        got = run_ns(gpu, xin, tdt(in_dt), tdt(compute), tdt(out_dt), MUON_ABC, 5, EPS)
        tol = TOL[compute] if out_dt == "f32" else max(TOL[compute], 2e-2)
        for x, u in zip(xin, got):
            e = rel_err(u, oracle.ns_orthogonalize(x, *MUON_ABC, 5, EPS))
            assert e <= tol, (in_dt, out_dt, x.shape, e)


def test_ns_in_place(gpu):
    import torch
    from matrix_optimizers_sharded_amd import ns_orthogonalize
    x = gaussian((200, 600), 9)
    t = to_dev_f32(x, gpu)
    ns_orthogonalize([t], [t], *MUON_ABC, 3, EPS, compute=torch.float32)
    torch.cuda.synchronize()
    assert rel_err(host_f32(t), oracle.ns_orthogonalize(x, *MUON_ABC, 3, EPS)) <= 1e-4


def test_textbook_quintic_bf16(gpu):
    import torch
    shapes = [(512, 768), (768, 512)]
    grads = [gaussian(s, 400 + i, 0.02) for i, s in enumerate(shapes)]
    moms = [gaussian(s, 500 + i, 0.02) for i, s in enumerate(shapes)]
    gm, gu = run_muon(gpu, grads, moms, torch.float32, torch.bfloat16, torch.float32, BETA,
                      TEXTBOOK_QUINTIC_ABC, 5, EPS)
    worst = check_muon(grads, moms, gm, gu, "bf16", TEXTBOOK_QUINTIC_ABC, 5, label="textbook quintic bf16")
    assert worst < 5e-3


@pytest.mark.parametrize("compute", ["f32", "bf16"])
def test_textbook_cubic(gpu, compute):
    """c = 0 (B' = aI + bA, the cubic iteration): both product paths, several
    256-tiles per matrix."""
    import torch
    shapes = [(512, 768), (768, 512), (200, 300)]
    grads = [gaussian(s, 430 + i, 0.02) for i, s in enumerate(shapes)]
    moms = [gaussian(s, 530 + i, 0.02) for i, s in enumerate(shapes)]
    dt = torch.float32 if compute == "f32" else torch.bfloat16
    gm, gu = run_muon(gpu, grads, moms, torch.float32, dt, torch.float32, BETA, TEXTBOOK_CUBIC_ABC, 5, EPS)
    check_muon(grads, moms, gm, gu, compute, TEXTBOOK_CUBIC_ABC, 5, label=f"textbook cubic {compute}")


def test_zero_matrix_gives_zero(gpu):
    import torch
    z = np.zeros((300, 500), np.float32)
    for compute in (torch.float32, torch.bfloat16):
        gm, gu = run_muon(gpu, [z], [z], torch.float32, compute, torch.float32, BETA, MUON_ABC, 5, EPS)
        assert np.all(gu[0] == 0) and np.all(gm[0] == 0)


@pytest.mark.parametrize("scale", [2.0 ** 70, 2.0 ** -70])
def test_extreme_input_scales(gpu, scale):
    """Inputs near the fp32 range ends: at 2^70 the squares (2^140) overflow fp32, so
    the Frobenius sum must not be formed in fp32; at 2^-70 the norm falls far below
    eps and X0 = x / (|x|_F + eps) stays tiny.  Both must follow the oracle, on both
    product paths (m = 300 on 256 x 256 tiles, m = 200 on 32 x 32 blocks)."""
    import torch
    shapes = [(300, 520), (520, 300), (200, 520), (520, 200)]
    xs = [(gaussian(s, 700 + i) * np.float32(scale)).astype(np.float32) for i, s in enumerate(shapes)]
    assert all(np.isfinite(x).all() for x in xs)
    say(f"extreme scale 2^{int(np.log2(scale))}")
    for compute in ("f32", "bf16"):
        got = run_ns(gpu, xs, tdt("f32"), tdt(compute), tdt("f32"), MUON_ABC, 5, EPS)
        for x, u in zip(xs, got):
            assert np.isfinite(u).all()
            e = rel_err(u, oracle.ns_orthogonalize(x, *MUON_ABC, 5, EPS))
            assert e <= TOL[compute], (compute, x.shape, e)


def test_first_product_scaling_range(gpu):
    """The first pass writes the operand unscaled and the first products apply the
    Frobenius factor, unless the norm lies outside [2^-20, 2^40]; then the operand is
    rewritten scaled.  One batch holds matrices just inside and just outside both
    ends (norms about 2^-19.4, 2^-21.4, 2^39.6, 2^40.6), so both routes run side by
    side in one call and each must follow the oracle, on both product paths (m = 300
    on 256 x 256 tiles, m = 200 on 32 x 32 blocks)."""
    import torch
    shapes = [(300, 520), (520, 300), (300, 520), (520, 300)]
    exps = [-28, -30, 31, 32]   # the unit Gaussians have norm about 2^8.6
    shapes = shapes + [(200, 520), (520, 200), (200, 520), (520, 200)]
    exps = exps + [-28, -30, 31, 32]
    xs = [(gaussian(s, 720 + i) * np.float32(2.0 ** e)).astype(np.float32) for i, (s, e) in enumerate(zip(shapes, exps))]
    norms = [np.log2(np.linalg.norm(x.astype(np.float64))) for x in xs]
    for q in (0, 4):
        assert norms[q] > -20 > norms[q + 1] and norms[q + 2] < 40 < norms[q + 3], norms
    say(f"first-product scaling, log2 norms {[round(v, 2) for v in norms]}")
    for compute in ("f32", "bf16"):
        got = run_ns(gpu, xs, tdt("f32"), tdt(compute), tdt("f32"), MUON_ABC, 5, EPS)
        for x, u in zip(xs, got):
            e = rel_err(u, oracle.ns_orthogonalize(x, *MUON_ABC, 5, EPS))
            assert e <= TOL[compute], (compute, x.shape, e)
    # the momentum step too: G = x, M = 0 makes the new momentum x itself
    zeros = [np.zeros_like(x) for x in xs]
    for compute in (torch.float32, torch.bfloat16):
        gm, gu = run_muon(gpu, xs, zeros, torch.float32, compute, torch.float32, BETA, MUON_ABC, 5, EPS)
        check_muon(xs, zeros, gm, gu, "f32" if compute == torch.float32 else "bf16", MUON_ABC, 5,
                   label="first-product scaling")


def _workload_inputs(wid):
    ins = [host_matrix(wid, i) for i in range(WORKLOADS[wid].count)]
    return [d["grad"] for d in ins], [d["mom"] for d in ins]


def test_125m_class_owner_set_bf16(gpu):
    """All 72 matrices of the 125M-class owner set in one batched call."""
    import torch
    w = WORKLOADS[2]
    say("workload 125m-class, 72 matrices, bf16 grads, bf16 compute")
    grads, moms = _workload_inputs(2)
    gm, gu = run_muon(gpu, grads, moms, torch.bfloat16, torch.bfloat16, torch.bfloat16, BETA, MUON_ABC,
                      w.iters, EPS)
    check_muon(grads, moms, gm, gu, "bf16", MUON_ABC, w.iters, label="125m-class")


def test_125m_class_fp32_grads_fp32_compute(gpu):
    import torch
    w = WORKLOADS[2]
    grads, moms = _workload_inputs(2)
    idx = [0, 4, 5]
    grads, moms = [grads[i] for i in idx], [moms[i] for i in idx]
    gm, gu = run_muon(gpu, grads, moms, torch.float32, torch.float32, torch.float32, BETA, MUON_ABC,
                      w.iters, EPS)
    check_muon(grads, moms, gm, gu, "f32", MUON_ABC, w.iters, label="125m-class fp32")


def test_deterministic_and_batch_invariant(gpu):
    import torch
    shapes = [(768, 768), (768, 3072), (3072, 768), (300, 200)]
    grads = [bf16_round(gaussian(s, 600 + i, 0.02))[1] for i, s in enumerate(shapes)]
    moms = [gaussian(s, 700 + i, 0.02) for i, s in enumerate(shapes)]
    run = lambda g, m: run_muon(gpu, g, m, torch.bfloat16, torch.bfloat16, torch.bfloat16, BETA, MUON_ABC, 5, EPS)
    m1, u1 = run(grads, moms)
    m2, u2 = run(grads, moms)
    for a, b in zip(u1, u2):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    for i in range(len(shapes)):
        mi, ui = run([grads[i]], [moms[i]])
        np.testing.assert_array_equal(ui[0].view(np.uint32), u1[i].view(np.uint32))
        np.testing.assert_array_equal(mi[0].view(np.uint32), m1[i].view(np.uint32))


def test_small_matrix_kernel_equals_the_plain_kernel(gpu):
    """bf16 SYRK / POLY launches whose matrices all have m <= 1024 run on the kernel's
    small-matrix instantiation (a diagonal tile loads its row panel once and reads
    both operands from it); a launch holding any larger matrix runs the plain one.  Both compute the same sums in the
    same order, so the small matrices' results must be equal bit for bit whether they
    run alone or beside a 2100-row matrix.  The no-allocation entry point keeps each
    call in one launch per product (no two-stream halves), so every matrix of a call
    shares that call's instantiation.  The large matrix is ragged (2100 x 2700: the
    last tile row and column are partial), so the plain kernel's edge tiles are
    checked against the oracle as well."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched_noalloc
    small = [(768, 768), (600, 1000), (1000, 600), (1000, 1800), (1024, 2304)]
    big = (2100, 2700)
    shapes = small + [big]
    grads = [bf16_round(gaussian(s, 1600 + i, 0.02))[1] for i, s in enumerate(shapes)]
    moms = [gaussian(s, 1700 + i, 0.02) for i, s in enumerate(shapes)]

    def run(idx):
        g = [to_dev_bf16(f32_to_bf16_bits(grads[i]), gpu) for i in idx]
        m = [to_dev_f32(moms[i], gpu) for i in idx]
        o = [torch.empty(shapes[i], dtype=torch.bfloat16, device=gpu) for i in idx]
        torch.cuda.synchronize()
        muon_step_batched_noalloc(g, m, o, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16)
        torch.cuda.synchronize()
        return [host_f32(x) for x in m], [host_f32(x) for x in o]

    say("small-matrix kernel: the small set alone, then beside a ragged 2100-row matrix")
    m_small, u_small = run(range(len(small)))
    m_mixed, u_mixed = run(range(len(shapes)))
    for i, sh in enumerate(small):
        np.testing.assert_array_equal(u_small[i].view(np.uint32), u_mixed[i].view(np.uint32),
                                      err_msg=f"U of {sh}")
        np.testing.assert_array_equal(m_small[i].view(np.uint32), m_mixed[i].view(np.uint32),
                                      err_msg=f"momentum of {sh}")
    # and the small-matrix kernel's results stay within the oracle's bar
    few = [0, 1, 2]
    check_muon([grads[i] for i in few], [moms[i] for i in few], [m_small[i] for i in few],
               [u_small[i] for i in few], "bf16", MUON_ABC, 5, label="small-matrix kernel")
    k = len(small)
    check_muon([grads[k]], [moms[k]], [m_mixed[k]], [u_mixed[k]], "bf16", MUON_ABC, 5,
               label="plain kernel, ragged 2100 x 2700")


def test_staged_output_with_edge_tiles(gpu):
    """The last product writes bf16 U through LDS as whole row pieces on blocks wholly
    inside the matrix when U's rows are 16-byte aligned, and element by element
    elsewhere.  These shapes have aligned rows (cols a multiple of 8) but sizes off
    the 256 grid, so one matrix mixes both paths, untransposed (wide) and transposed
    (tall); two more have rows only 8-byte aligned, which take the element path
    throughout."""
    import torch
    shapes = [(1000, 1288), (1288, 1000), (520, 2056), (2056, 520), (776, 1004), (1004, 772)]
    grads = [bf16_round(gaussian(s, 1800 + i, 0.02))[1] for i, s in enumerate(shapes)]
    moms = [gaussian(s, 1900 + i, 0.02) for i, s in enumerate(shapes)]
    say("staged U with edge tiles: " + ", ".join(f"{r}x{c}" for r, c in shapes))
    gm, gu = run_muon(gpu, grads, moms, torch.bfloat16, torch.bfloat16, torch.bfloat16, BETA, MUON_ABC, 5, EPS)
    check_muon(grads, moms, gm, gu, "bf16", MUON_ABC, 5, label="staged U, edge tiles")
    # the same U written one element off 16-byte alignment takes the element path
    # everywhere: both paths round the same values, so U must be equal bit for bit
    from matrix_optimizers_sharded_amd import muon_step_batched
    g_dev = [to_dev_bf16(f32_to_bf16_bits(g), gpu) for g in grads]
    m_dev = [to_dev_f32(m, gpu) for m in moms]
    flat = [torch.empty(r * c + 8, dtype=torch.bfloat16, device=gpu) for r, c in shapes]
    outs = [f[1:1 + r * c].view(r, c) for f, (r, c) in zip(flat, shapes)]
    assert all(o.data_ptr() % 16 != 0 for o in outs)
    torch.cuda.synchronize()
    muon_step_batched(g_dev, m_dev, outs, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16)
    torch.cuda.synchronize()
    for i, sh in enumerate(shapes):
        np.testing.assert_array_equal(host_f32(outs[i]).view(np.uint32), gu[i].view(np.uint32),
                                      err_msg=f"U of {sh}: staged against element by element")


def test_split_batch_follows_the_callers_stream(gpu):
    """A batch with few rounds of tiles per launch runs its products as two halves,
    one on the caller's stream and one on the library's second stream.  Inputs
    written on the caller's stream right before the call (behind a spin kernel, so
    they land late) must be what the second half reads, and the caller's next work
    must see both halves' outputs."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched
    shapes = [(768, 768), (768, 3072), (3072, 768), (768, 768), (512, 1024)]
    grads = [bf16_round(gaussian(s, 800 + i, 0.02))[1] for i, s in enumerate(shapes)]
    moms = [gaussian(s, 900 + i, 0.02) for i, s in enumerate(shapes)]
    m_ref, u_ref = run_muon(gpu, grads, moms, torch.bfloat16, torch.bfloat16, torch.bfloat16, BETA, MUON_ABC, 5,
                            EPS)
    g_src = [to_dev_bf16(f32_to_bf16_bits(g), gpu) for g in grads]
    m_src = [to_dev_f32(m, gpu) for m in moms]
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=gpu)
    with torch.cuda.stream(s):
        g_dev = [torch.zeros_like(t) for t in g_src]
        m_dev = [torch.zeros_like(t) for t in m_src]
        outs = [torch.zeros(sh, dtype=torch.bfloat16, device=gpu) for sh in shapes]
        torch.cuda._sleep(50_000_000)
        for d, t in zip(g_dev + m_dev, g_src + m_src):
            d.copy_(t)
        muon_step_batched(g_dev, m_dev, outs, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16)
        got = [o.clone() for o in outs]
    s.synchronize()
    for i in range(len(shapes)):
        np.testing.assert_array_equal(host_f32(got[i]).view(np.uint32), u_ref[i].view(np.uint32))
        np.testing.assert_array_equal(host_f32(m_dev[i]).view(np.uint32), m_ref[i].view(np.uint32))


def test_split_batches_from_two_threads(gpu):
    """Two host threads, each with its own torch stream, call the split path at the
    same time (ctypes releases the GIL, and both calls share the library's second
    stream and its fork/join events): every call's results equal the same batch run
    alone."""
    import threading
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched
    sets = [[(768, 768), (768, 2048), (1024, 512)], [(512, 1536), (768, 768), (640, 1280)]]
    inputs, refs = [], []
    for t, shapes in enumerate(sets):
        grads = [bf16_round(gaussian(s, 1400 + 10 * t + i, 0.02))[1] for i, s in enumerate(shapes)]
        moms = [gaussian(s, 1500 + 10 * t + i, 0.02) for i, s in enumerate(shapes)]
        inputs.append((shapes, grads, moms))
        refs.append(run_muon(gpu, grads, moms, torch.bfloat16, torch.bfloat16, torch.bfloat16, BETA, MUON_ABC, 5,
                             EPS))
    got, errors = {}, []

    def worker(t):
        try:
            shapes, grads, moms = inputs[t]
            s = torch.cuda.Stream(device=gpu)
            with torch.cuda.stream(s):
                g_dev = [to_dev_bf16(f32_to_bf16_bits(g), gpu) for g in grads]
                m0 = [to_dev_f32(m, gpu) for m in moms]
                m_dev = [torch.empty_like(m) for m in m0]
                outs = [torch.empty(sh, dtype=torch.bfloat16, device=gpu) for sh in shapes]
                runs = []
                for _ in range(4):
                    for m, m_init in zip(m_dev, m0):
                        m.copy_(m_init)
                    muon_step_batched(g_dev, m_dev, outs, BETA, *MUON_ABC, 5, EPS, compute=torch.bfloat16)
                    runs.append(([o.clone() for o in outs], [m.clone() for m in m_dev]))
            s.synchronize()
            got[t] = [([host_f32(o) for o in us], [host_f32(m) for m in ms]) for us, ms in runs]
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(len(sets))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(len(sets)):
        m_ref, u_ref = refs[t]
        for r, (us, ms) in enumerate(got[t]):
            for i in range(len(sets[t])):
                np.testing.assert_array_equal(us[i].view(np.uint32), u_ref[i].view(np.uint32),
                                              err_msg=f"thread {t} call {r} matrix {i}: U")
                np.testing.assert_array_equal(ms[i].view(np.uint32), m_ref[i].view(np.uint32),
                                              err_msg=f"thread {t} call {r} matrix {i}: momentum")


def test_profile_busy_time_merges_overlapping_halves(gpu):
    """mo_profile_end's busy time is the union of a kind's launch intervals: for the
    products of a split batch (two halves on two streams) it lies between the longest
    single launch and the sum of all of them; for kinds launched once per step on one
    stream it equals the sum."""
    import torch
    import matrix_optimizers_sharded_amd as mo
    shapes = [(768, 768), (768, 3072), (3072, 768), (768, 768)]
    grads = [to_dev_bf16(f32_to_bf16_bits(bf16_round(gaussian(s, 1600 + i, 0.02))[1]), gpu)
             for i, s in enumerate(shapes)]
    moms = [to_dev_f32(gaussian(s, 1700 + i, 0.02), gpu) for i, s in enumerate(shapes)]
    outs = [torch.empty(s, dtype=torch.bfloat16, device=gpu) for s in shapes]
    ws = mo.Workspace(gpu)
    mo.muon_step_batched(grads, moms, outs, BETA, *MUON_ABC, 5, EPS, workspace=ws)
    torch.cuda.synchronize()
    mo.profile_begin()
    for _ in range(3):
        mo.muon_step_batched(grads, moms, outs, BETA, *MUON_ABC, 5, EPS, workspace=ws)
    torch.cuda.synchronize()
    k = mo.profile_end()
    say(f"profile: {k}")
    for name in ("ns_syrk", "ns_poly", "ns_apply"):
        launches, total, busy = k[name]
        assert launches == 3 * 5 * 2, (name, launches)          # 3 calls x 5 iterations x 2 halves
        assert busy <= total * (1 + 1e-6), (name, busy, total)
        assert busy >= total / launches, (name, busy, total)
    launches, total, busy = k["momentum_prep"]
    assert launches == 3 and abs(busy - total) <= 1e-3 * total, (busy, total)


def test_tall_is_transpose_of_wide(gpu):
    import torch
    g = gaussian((200, 520), 5)
    m = gaussian((200, 520), 6)
    _, uw = run_muon(gpu, [g], [m], torch.float32, torch.float32, torch.float32, BETA, MUON_ABC, 5, EPS)
    _, ut = run_muon(gpu, [g.T.copy()], [m.T.copy()], torch.float32, torch.float32, torch.float32, BETA,
                     MUON_ABC, 5, EPS)
    assert rel_err(ut[0], uw[0].T) <= 1e-5
