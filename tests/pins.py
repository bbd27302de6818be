"""Pin checks for the oracle: each compares an oracle function with something other
than itself (a closed form, a library routine, exact rational arithmetic or brute
force).  They take the function under test as an argument so that the mutation
test can run the same checks on oracle copies with planted mistakes.
"""

from fractions import Fraction

import numpy as np
import scipy.linalg


def random_orthogonal(rng, n):
    q, r = np.linalg.qr(rng.standard_normal((n, n)))
    return q * np.sign(np.diag(r))[None, :]


def scalar_poly_iterate(sigma, a, b, c, iters):
    """p^k(sigma) with p(s) = a s + b s^3 + c s^5, on scalars.

    If X = U diag(s) V^T then A = X X^T = U diag(s^2) U^T, bA + cA^2 =
    U diag(b s^2 + c s^4) U^T and aX + (bA + cA^2) X = U diag(p(s)) V^T, so k steps
    map each singular value through p k times and keep U and V."""
    a, b, c = (float(np.float32(v)) for v in (a, b, c))
    s = np.array(sigma, dtype=np.float64)
    for _ in range(iters):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def closed_form_error(ns_fn, shape, abc, iters, seed=0, orient=True):
    """Relative Frobenius error of ns_fn(X0) against U diag(p^k(sigma)) V^T for an X0
    built from chosen singular vectors and values."""
    rng = np.random.default_rng(seed)
    r, s = shape
    k = min(r, s)
    U = random_orthogonal(rng, r)[:, :k]
    V = random_orthogonal(rng, s)[:, :k]
    sigma = np.sort(rng.uniform(0.02, 1.0, size=k))[::-1]
    x0 = (U * sigma) @ V.T
    want = (U * scalar_poly_iterate(sigma, *abc, iters)) @ V.T
    got = ns_fn(x0, *abc, iters) if orient else ns_fn(x0, *abc, iters, orient=False)
    if got.shape != want.shape:
        return np.inf
    return np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)


def polar_error(ns_fn, shape, abc, iters, seed=1):
    """Relative error of ns_fn on a normalised Gaussian matrix against the polar
    factor from scipy.linalg.polar (for convergent coefficients)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    x0 = x / np.linalg.norm(x)
    r, s = shape
    if r >= s:
        upol, _ = scipy.linalg.polar(x0, side="right")
    else:
        upol, _ = scipy.linalg.polar(x0.T, side="right")
        upol = upol.T
    got = ns_fn(x0, *abc, iters)
    return np.linalg.norm(got - upol) / np.linalg.norm(upol)


def exact_fma_f32(beta, m, g):
    """Correctly rounded float32 of beta*m + g, by exact rational arithmetic and a
    search over neighbouring float32 values (ties to even significand)."""
    exact = Fraction(float(np.float32(beta))) * Fraction(float(np.float32(m))) + Fraction(float(g))
    r0 = np.float32(float(exact))
    cands = [r0]
    for d in (np.float32(-np.inf), np.float32(np.inf)):
        c = r0
        for _ in range(2):
            c = np.nextafter(c, d)
            cands.append(c)
    best = None
    for c in cands:
        dist = abs(Fraction(float(c)) - exact)
        key = (dist, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def brute_pack(values):
    """Bits by a Python loop over values; words by building each word's binary
    string most-significant bit first and parsing it."""
    bits = ["1" if v >= 0 else "0" for v in values]   # NaN >= 0 is False
    words = []
    for w in range(0, len(bits), 32):
        chunk = bits[w:w + 32] + ["0"] * (32 - len(bits[w:w + 32]))
        words.append(int("".join(reversed(chunk)), 2))
    return np.array(words, dtype=np.uint32)


def brute_vote(packed_rows, numel):
    """Per element, a Python count of +1 and -1 votes; tie -> +1."""
    M = len(packed_rows)
    out_bits, sums = [], []
    for i in range(numel):
        plus = sum((int(row[i // 32]) >> (i % 32)) & 1 for row in packed_rows)
        total = plus - (M - plus)
        sums.append(total)
        out_bits.append(1.0 if total >= 0 else -1.0)
    return brute_pack(out_bits), np.array(sums, dtype=np.int64)
