"""Owner planner: the oracle's longest-processing-time rule pinned to brute-force
optimal assignments (Graham's bound) and to hand-checkable cases, and the library's
host-side planner (C ABI, no GPU needed) equal to the oracle assignment for
assignment."""

import itertools
import random

import pytest

import oracle
from matrix_optimizers_sharded_amd import binding, plan_owners
from matrix_optimizers_sharded_amd.workloads import WORKLOADS


def random_shapes(rng, k):
    dims = [128, 256, 384, 768, 1024, 2048]
    return [(rng.choice(dims), rng.choice(dims)) for _ in range(k)]


def test_work_is_the_flop_count():
    assert oracle.ns_work(4096, 11008, 5) == oracle.ns_polynomial_flops(4096, 11008, 5)
    assert oracle.ns_work(11008, 4096, 5) == oracle.ns_work(4096, 11008, 5)
    assert oracle.ns_work(3, 5, 1) == 3 * 3 * 5 + 27 + 2 * 3 * 3 * 5


def test_hand_case():
    shapes = [(1, 8), (1, 7), (1, 6), (1, 5), (1, 4)]   # m = 1: work = iters * (3n + 1)
    owners, load_w, _ = oracle.lpt_owners(shapes, 2, 1)
    works = [oracle.ns_work(r, c, 1) for r, c in shapes]
    assert works == [25.0, 22.0, 19.0, 16.0, 13.0]
    # 25 -> r0; 22 -> r1; 19 -> r1 (22 < 25); 16 -> r0 (25 < 41); 13 -> r0 (41 = 41,
    # r0 holds 8+5 = 13 elements of bytes vs r1's 7+6 = 13: equal -> lower rank)
    assert owners == [0, 1, 1, 0, 0]
    assert load_w == [54.0, 41.0]


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound_of_brute_force(seed):
    rng = random.Random(seed)
    ranks = rng.choice([2, 3])
    shapes = random_shapes(rng, rng.randint(1, 7))
    owners, load_w, _ = oracle.lpt_owners(shapes, ranks, 5)
    works = [oracle.ns_work(r, c, 5) for r, c in shapes]
    got = oracle.makespan(owners, works, ranks)
    opt = oracle.optimal_makespan(works, ranks)
    assert got >= opt - 1e-6
    assert got <= (4.0 / 3.0 - 1.0 / (3 * ranks)) * opt + 1e-6
    assert abs(sum(load_w) - sum(works)) < 1e-6 * sum(works)


def test_fewer_matrices_than_ranks_get_distinct_owners():
    shapes = [(256, 256), (512, 768), (1024, 1024)]
    owners, _, _ = oracle.lpt_owners(shapes, 8, 5)
    assert sorted(owners) == [0, 1, 2]


def test_identical_matrices_spread_evenly():
    owners, load_w, load_b = oracle.lpt_owners([(512, 512)] * 10, 4, 5)
    counts = [owners.count(r) for r in range(4)]
    assert counts == [3, 3, 2, 2]
    assert max(load_b) - min(load_b) == 512 * 512 * 4.0


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


@pytest.mark.parametrize("seed", range(25))
def test_library_planner_equals_oracle(lib, seed):
    rng = random.Random(100 + seed)
    ranks = rng.choice([1, 2, 3, 4, 8, 16])
    shapes = random_shapes(rng, rng.randint(1, 40))
    if seed % 5 == 0:
        shapes = shapes + shapes[:5]          # exact ties in work and bytes
    iters = rng.choice([0, 1, 5])
    bpe = rng.choice([0.0, 2.0, 10.0])
    got_o, got_w, got_b = plan_owners(shapes, ranks, iters, bpe)
    want_o, want_w, want_b = oracle.lpt_owners(shapes, ranks, iters, bpe)
    assert got_o == want_o
    assert got_w == pytest.approx(want_w, rel=1e-12)
    assert got_b == pytest.approx(want_b, rel=1e-12)


def test_library_planner_on_the_7b_owner_set(lib):
    shapes = WORKLOADS[4].shapes
    for ranks in (1, 2, 8, 64):
        got_o, got_w, _ = plan_owners(shapes, ranks, 5, 10.0)
        want_o, want_w, _ = oracle.lpt_owners(shapes, ranks, 5, 10.0)
        assert got_o == want_o
        total = sum(oracle.ns_work(r, c, 5) for r, c in shapes)
        assert sum(got_w) == pytest.approx(total)
        # LPT bound against the trivial lower bound max(total / R, largest job)
        lower = max(total / ranks, max(oracle.ns_work(r, c, 5) for r, c in shapes))
        assert max(got_w) <= (4.0 / 3.0) * lower * 1.000001


def test_library_planner_rejects_bad_arguments(lib):
    import ctypes
    I64 = ctypes.c_int64 * 1
    own = (ctypes.c_int32 * 1)()
    assert lib.mo_plan_owners(I64(4), I64(4), 1, 0, 5, 4.0, own, None, None) == -1
    assert lib.mo_plan_owners(I64(0), I64(4), 1, 2, 5, 4.0, own, None, None) == -1
    assert lib.mo_plan_owners(I64(4), I64(4), 1, 2, -1, 4.0, own, None, None) == -1
    assert lib.mo_plan_owners(I64(4), I64(4), 1, 2, 5, float("nan"), own, None, None) == -1
    assert lib.mo_plan_owners(None, None, 0, 2, 5, 4.0, None, None, None) == 0
