"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pins catch every one.  This shows the pins constrain the oracle: a dropped term,
a wrong sign, a transposed operand or a wrong bit order all fail."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import MUON_ABC, TEXTBOOK_QUINTIC_ABC
from pins import closed_form_error, polar_error, brute_pack, brute_vote


def _ns(step):
    def ns(x, a, b, c, iters, orient=True):
        X = np.array(x, dtype=np.float64)
        flip = orient and X.shape[0] > X.shape[1]
        if flip:
            X = X.T
        for _ in range(iters):
            X = step(X, a, b, c)
        return X.T if flip else X
    return ns


MUTANTS = {
    "drop_cA2": lambda X, a, b, c: a * X + (b * (X @ X.T)) @ X,
    "flip_b": lambda X, a, b, c: a * X + (-b * (X @ X.T) + c * (X @ X.T) @ (X @ X.T)) @ X,
    "drop_aX": lambda X, a, b, c: (b * (X @ X.T) + c * (X @ X.T) @ (X @ X.T)) @ X,
    "gram_transposed": lambda X, a, b, c: a * X + (b * (X.T @ X) + c * (X.T @ X) @ (X.T @ X)) @ X,
    "cubic_power": lambda X, a, b, c: a * X + (b * (X @ X.T) + c * (X @ X.T)) @ X,
    "swap_b_c": lambda X, a, b, c: a * X + (c * (X @ X.T) + b * (X @ X.T) @ (X @ X.T)) @ X,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_ns_mutants_fail_a_pin(name):
    ns = _ns(MUTANTS[name])
    errs = []
    for shape in [(16, 8), (8, 16), (12, 12)]:
        try:
            errs.append(closed_form_error(ns, shape, MUON_ABC, 3, seed=1))
        except ValueError:
            errs.append(np.inf)
        try:
            errs.append(polar_error(ns, shape, TEXTBOOK_QUINTIC_ABC, 14))
        except ValueError:
            errs.append(np.inf)
    assert max(errs) > 1e-6, errs


def test_correct_oracle_passes_the_same_checks():
    for shape in [(16, 8), (8, 16), (12, 12)]:
        assert closed_form_error(oracle.newton_schulz, shape, MUON_ABC, 3, seed=1) < 1e-12
        assert polar_error(oracle.newton_schulz, shape, TEXTBOOK_QUINTIC_ABC, 14) < 1e-12


def test_no_transpose_back_fails():
    def ns(x, a, b, c, iters, orient=True):
        X = np.array(x, dtype=np.float64)
        if X.shape[0] > X.shape[1]:
            X = X.T
        for _ in range(iters):
            A = X @ X.T
            X = a * X + (b * A + c * A @ A) @ X
        return X        # forgot to transpose back
    assert closed_form_error(ns, (16, 8), MUON_ABC, 3) == np.inf


def test_pack_and_vote_mutants_fail_brute_force():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(70)
    v[3] = 0.0
    v[5] = -0.0
    msb_first = lambda u: np.array(
        [int("".join("1" if x >= 0 else "0" for x in (list(u[i:i + 32]) + [-1] * (32 - len(u[i:i + 32])))), 2)
         for i in range(0, len(u), 32)], dtype=np.uint32)
    strict_sign = lambda u: oracle.pack_bits((np.asarray(u) > 0).astype(np.uint8))
    for mutant in (msb_first, strict_sign):
        assert not np.array_equal(mutant(v), brute_pack(v))
    packed = np.stack([oracle.sign_pack(rng.standard_normal(70)) for _ in range(4)])
    ties_negative = lambda p, n: oracle.pack_bits((oracle.majority_vote(p, n)[1] > 0).astype(np.uint8))
    assert not np.array_equal(ties_negative(packed, 70), brute_vote(list(packed), 70)[0])
