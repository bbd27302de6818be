"""fp64 oracle for the owner-local Muon step: momentum, Frobenius scaling, quintic
Newton-Schulz.  TEST INFRASTRUCTURE ONLY (see the package docstring): the product
path never imports this module.

Every function works on one matrix at a time, in numpy float64, with numpy's BLAS
matmul as the only library step.  There is no blocking, fusion or reordering beyond
what the definitions below state.

Scalars (beta, a, b, c, eps) are taken as the float32 values the GPU library
receives and widened exactly to float64, so both sides start from identical numbers.
"""

import numpy as np


def _f32_scalar(v):
    """The float32 value a caller-supplied scalar becomes at the C boundary, widened
    exactly to float64."""
    return float(np.float32(v))


def momentum_update(grad, mom, beta):
    """Heavy-ball momentum M <- beta*M + G, in float64.

    "Riepilogo Tecnico: SignMuon", section 2, distributed flow item 1: each worker
    takes its stochastic gradient G_t and updates its local momentum M_{t+1}; section
    4 "Memoria e Sovraccarico": a single momentum buffer, as in SGD.  The pages print
    no formula; the reading taken is the SGD heavy-ball form beta*M + G (no
    dampening, no Nesterov look-ahead), and the new M is what Newton-Schulz sees.
    """
    b = _f32_scalar(beta)
    return b * np.asarray(mom, dtype=np.float64) + np.asarray(grad, dtype=np.float64)


def momentum_state_fp32(grad, mom, beta):
    """The float32 momentum state a single correctly rounded fused multiply-add
    fl32(beta*M + G) leaves behind, for float32 M and float32/bf16 G.

    beta*M is exact in float64 (24-bit by 24-bit significands).  The sum with G is
    formed in float64 together with its exact rounding error (Knuth's TwoSum), and
    the pair is rounded once to float32: a float64 sum that lands exactly on a
    float32 rounding midpoint is resolved by the sign of the error term, and only
    an exact midpoint falls back to ties-to-even.
    """
    b = _f32_scalar(beta)
    m = np.asarray(mom, dtype=np.float32).astype(np.float64)
    g = np.asarray(grad, dtype=np.float64)
    p = b * m                      # exact
    s = p + g                      # rounded to float64
    bv = s - p
    e = (p - (s - bv)) + (g - bv)  # exact error: p + g == s + e
    r = s.astype(np.float32)       # round-to-nearest-even
    r64 = r.astype(np.float64)
    toward = np.where(s > r64, np.float32(np.inf), np.float32(-np.inf))
    other = np.nextafter(r, toward)
    mid = (r64 + other.astype(np.float64)) * 0.5   # exact: a 25-bit value
    tie = (s != r64) & (s == mid) & (e != 0)
    if np.any(tie):
        up = np.maximum(r, other)
        down = np.minimum(r, other)
        r = np.where(tie, np.where(e > 0, up, down), r)
    return r


def frobenius_normalize(m, eps):
    """X0 = M / (||M||_F + eps), one scalar per matrix.

    "Riepilogo Tecnico: SignMuon", section 4 (nanoGPT) names Frobenius versus
    spectral scaling; section 3 requires an update whose spectral norm is at most 1,
    which dividing by the Frobenius norm guarantees for the input of the iteration
    (sigma_max <= ||M||_F).  eps is a reading (the pages give none): it keeps a zero
    matrix finite, and a zero matrix maps to zero.
    """
    m = np.asarray(m, dtype=np.float64)
    return m / (np.sqrt(np.sum(m * m)) + _f32_scalar(eps))


def newton_schulz(x, a, b, c, iters, orient=True):
    """k quintic Newton-Schulz steps X <- aX + (bA + cA^2)X with A = X X^T.

    "Riepilogo Tecnico: SignMuon", section 2, core mechanism item 1: the polar
    direction of the momentum is approximated locally by Newton-Schulz iteration,
    which orthogonalises it; section 4 (nanoGPT): often a single iteration is
    enough, so iters is a parameter and iters == 0 returns the input.  The quintic
    form and (a, b, c) as parameters are readings; the pages print neither.

    orient=True works on the transpose when the matrix has more rows than columns,
    so A is the smaller Gram matrix (min(r,s) squared); the result is transposed
    back.  In exact arithmetic p(XX^T)X == X p(X^T X), so this changes rounding
    only; orient=False runs the literal form on the matrix as given.
    """
    af, bf, cf = _f32_scalar(a), _f32_scalar(b), _f32_scalar(c)
    X = np.array(x, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a 2D matrix")
    flip = orient and X.shape[0] > X.shape[1]
    if flip:
        X = X.T
    for _ in range(int(iters)):
        A = X @ X.T
        B = bf * A + cf * (A @ A)
        X = af * X + B @ X
    if flip:
        X = X.T
    return np.ascontiguousarray(X)


def ns_orthogonalize(x, a, b, c, iters, eps, orient=True):
    """Frobenius-normalise, then run the Newton-Schulz iteration (no momentum)."""
    return newton_schulz(frobenius_normalize(x, eps), a, b, c, iters, orient)


def muon_step(grad, mom, beta, a, b, c, iters, eps, orient=True):
    """One owner-local Muon step on one whole matrix.

    "Riassunto Tecnico: MatrixFSDP", section "Metodologia", item 1: the owner rank
    holds the full 2D gradient after the reduction and runs the Newton-Schulz update
    locally, with no matrix communication.  Steps: momentum (float64), Frobenius
    scaling, k Newton-Schulz steps.

    Returns (new momentum as the float32 state a fused multiply-add leaves,
    U in float64).  The iteration starts from the unrounded float64 momentum.
    """
    m_new = momentum_update(grad, mom, beta)
    u = ns_orthogonalize(m_new, a, b, c, iters, eps, orient)
    return momentum_state_fp32(grad, mom, beta), u


def weight_update(weight, u, lr):
    """The owner's parameter update W - lr * U in float64.

    The form follows "Riepilogo Tecnico: SignMuon", distributed flow item 4
    (W_{t+1} = W_t - eta_t * direction), with the polar factor U itself as the Muon
    direction: the pages give no other scaling for Muon (reading S7).  lr is taken
    as the float32 value the caller passes."""
    return np.asarray(weight, dtype=np.float64) - _f32_scalar(lr) * np.asarray(u, dtype=np.float64)


def ns_polynomial_flops(rows, cols, iters):
    """Algorithmic flop count of the iteration on one r x s matrix: per step
    m^2 n (upper triangle of A = X X^T) + m^3 (A^2, symmetric) + 2 m^2 n (B X),
    with m = min(r, s), n = max(r, s).  Used by the CPU-baseline timing only."""
    m, n = min(rows, cols), max(rows, cols)
    return int(iters) * (3 * m * m * n + m ** 3)
