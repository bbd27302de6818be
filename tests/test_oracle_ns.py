"""Pins of the Newton-Schulz / momentum / scaling oracle against closed forms,
library routines and exact arithmetic (CPU only)."""

import numpy as np
import pytest

import oracle
from matrix_optimizers_sharded_amd.workloads import (
    MUON_ABC, TEXTBOOK_QUINTIC_ABC, TEXTBOOK_CUBIC_ABC, EPS)
from pins import (closed_form_error, polar_error, exact_fma_f32, scalar_poly_iterate,
                  random_orthogonal)

COEFFS = {"muon": MUON_ABC, "quintic": TEXTBOOK_QUINTIC_ABC, "cubic": TEXTBOOK_CUBIC_ABC}
SHAPES = [(64, 32), (32, 64), (48, 48), (7, 13), (13, 7), (1, 9), (9, 1), (1, 1)]


@pytest.mark.parametrize("name", sorted(COEFFS))
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("iters", [0, 1, 2, 5])
def test_singular_value_closed_form(name, shape, iters):
    err = closed_form_error(oracle.newton_schulz, shape, COEFFS[name], iters, seed=hash(shape) % 1000)
    assert err < 1e-12, err


@pytest.mark.parametrize("shape", [(64, 32), (32, 64), (40, 40), (5, 17)])
def test_literal_orientation_matches_closed_form(shape):
    # orient=False runs A = X X^T on the matrix as given, even when it is tall
    err = closed_form_error(oracle.newton_schulz, shape, MUON_ABC, 5, seed=3, orient=False)
    assert err < 1e-12, err


@pytest.mark.parametrize("shape", [(64, 32), (32, 64), (30, 30), (100, 7)])
def test_textbook_quintic_reaches_polar_factor(shape):
    assert polar_error(oracle.newton_schulz, shape, TEXTBOOK_QUINTIC_ABC, 14) < 1e-12


@pytest.mark.parametrize("shape", [(64, 32), (32, 64)])
def test_textbook_cubic_reaches_polar_factor(shape):
    assert polar_error(oracle.newton_schulz, shape, TEXTBOOK_CUBIC_ABC, 30) < 1e-12


def test_convergent_sets_keep_spectral_norm_at_most_one():
    # "Riepilogo Tecnico: SignMuon", section 3: update spectral norm at most 1.  For
    # the textbook sets p maps [0, 1] into [0, 1], so every iterate obeys it.
    rng = np.random.default_rng(7)
    for abc in (TEXTBOOK_QUINTIC_ABC, TEXTBOOK_CUBIC_ABC):
        for k in (1, 3, 8):
            x = rng.standard_normal((40, 24))
            u = oracle.ns_orthogonalize(x, *abc, k, EPS)
            assert np.linalg.norm(u, 2) <= 1.0 + 1e-12


def test_singular_values_follow_polynomial_on_gaussian_input():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 80))
    x0 = oracle.frobenius_normalize(x, EPS)
    u = oracle.newton_schulz(x0, *MUON_ABC, 5)
    s_in = np.linalg.svd(x0, compute_uv=False)
    s_out = np.sort(np.linalg.svd(u, compute_uv=False))
    want = np.sort(scalar_poly_iterate(s_in, *MUON_ABC, 5))
    np.testing.assert_allclose(s_out, want, rtol=1e-10, atol=1e-13)


def test_transpose_and_orthogonal_equivariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((24, 40))
    f = lambda m: oracle.ns_orthogonalize(m, *MUON_ABC, 5, EPS)
    np.testing.assert_allclose(f(x.T), f(x).T, rtol=0, atol=1e-12)
    Q, R = random_orthogonal(rng, 24), random_orthogonal(rng, 40)
    np.testing.assert_allclose(f(Q @ x @ R), Q @ f(x) @ R, rtol=0, atol=1e-11)


def test_special_cases():
    abc = MUON_ABC
    eps = float(np.float32(EPS))
    # zero matrix -> exactly zero
    z = oracle.ns_orthogonalize(np.zeros((6, 9)), *abc, 5, EPS)
    assert np.all(z == 0)
    # k = 0 returns the normalised input
    x = np.arange(12.0).reshape(3, 4) - 5
    np.testing.assert_array_equal(oracle.ns_orthogonalize(x, *abc, 0, EPS),
                                  x / (np.sqrt((x * x).sum()) + eps))
    # rank one u v^T: one singular value s/(s+eps), mapped through p^k
    u, v = np.array([1.0, 2.0, 2.0]), np.array([3.0, 4.0])
    x = np.outer(u, v)
    s = np.linalg.norm(u) * np.linalg.norm(v)
    sig = scalar_poly_iterate([s / (s + eps)], *abc, 5)[0]
    np.testing.assert_allclose(oracle.ns_orthogonalize(x, *abc, 5, EPS),
                               sig * np.outer(u / 3.0, v / 5.0), rtol=1e-13)
    # scaled identity
    n = 16
    got = oracle.ns_orthogonalize(np.eye(n), *abc, 3, EPS)
    sig = scalar_poly_iterate([1.0 / (np.sqrt(n) + eps)], *abc, 3)[0]
    np.testing.assert_allclose(got, sig * np.eye(n), rtol=1e-13, atol=1e-16)


def test_frobenius_normalize_closed_form():
    x = np.ones((3, 5))
    np.testing.assert_allclose(oracle.frobenius_normalize(x, 0.0), x / np.sqrt(15.0), rtol=1e-15)
    x = np.array([[3.0, 0.0], [0.0, 4.0]])
    np.testing.assert_allclose(oracle.frobenius_normalize(x, 0.0), x / 5.0, rtol=1e-15)
    # per-matrix scale invariance up to eps
    y = np.random.default_rng(2).standard_normal((8, 8))
    np.testing.assert_allclose(oracle.frobenius_normalize(1000.0 * y, EPS),
                               oracle.frobenius_normalize(y, EPS), rtol=1e-6)


def test_momentum_update_closed_form():
    g = np.array([[3.0, -1.0]])
    m = np.array([[2.0, 4.0]])
    np.testing.assert_array_equal(oracle.momentum_update(g, m, 0.5), [[4.0, 1.0]])
    # beta is taken as the float32 value the C boundary receives
    b32 = float(np.float32(0.95))
    np.testing.assert_array_equal(oracle.momentum_update(g, m, 0.95), b32 * m + g)


def test_momentum_state_matches_exact_rational_fma():
    rng = np.random.default_rng(9)
    m = rng.standard_normal(400).astype(np.float32)
    g = (rng.standard_normal(400) * rng.choice([1e-3, 1.0, 1e3], 400)).astype(np.float32)
    for beta in (0.95, 0.9, 0.5, 0.999):
        got = oracle.momentum_state_fp32(g, m, beta)
        want = np.array([exact_fma_f32(beta, mi, gi) for mi, gi in zip(m, g)], dtype=np.float32)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_momentum_state_resolves_false_float64_ties():
    # beta*M = 2^-24 - 2^-54 and G = 1 + 2^-23: the float64 sum rounds onto the
    # float32 midpoint 1 + 3*2^-24, where ties-to-even would round up to 1 + 2^-22;
    # the exact value lies below the midpoint, so the correct result is 1 + 2^-23.
    beta = np.float32(1 + 2.0 ** -15)
    m = np.array([2.0 ** -24 * (1 - 2.0 ** -15), -(2.0 ** -24) * (1 - 2.0 ** -15)], np.float32)
    g = np.array([1 + 2.0 ** -23, -(1 + 2.0 ** -23)], np.float32)
    got = oracle.momentum_state_fp32(g, m, beta)
    want = np.array([exact_fma_f32(beta, mi, gi) for mi, gi in zip(m, g)], dtype=np.float32)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(got, np.array([1 + 2.0 ** -23, -(1 + 2.0 ** -23)], np.float32))
    naive = (float(beta) * m.astype(np.float64) + g).astype(np.float32)
    assert naive[0] != got[0]   # the case really is a double-rounding trap


def test_muon_step_composes_momentum_and_ns():
    rng = np.random.default_rng(4)
    g = rng.standard_normal((10, 6)).astype(np.float32)
    m = rng.standard_normal((10, 6)).astype(np.float32)
    m_new, u = oracle.muon_step(g, m, 0.95, *MUON_ABC, 5, EPS)
    want_u = oracle.ns_orthogonalize(oracle.momentum_update(g, m, 0.95), *MUON_ABC, 5, EPS)
    np.testing.assert_array_equal(u, want_u)
    assert m_new.dtype == np.float32


def test_weight_update_is_w_minus_lr_u():
    w = np.array([[1.0, -2.0], [0.5, 0.0]])
    u = np.array([[0.5, 0.25], [-1.0, 2.0]])
    np.testing.assert_array_equal(oracle.weight_update(w, u, 0.5), [[0.75, -2.125], [1.0, -1.0]])
    # lr passes through float32 at the C boundary: 0.1f, not 0.1
    got = oracle.weight_update(np.zeros((1, 1)), np.ones((1, 1)), 0.1)
    assert got[0, 0] == -float(np.float32(0.1)) != -0.1
