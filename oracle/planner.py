"""Oracle for the owner planner.  TEST INFRASTRUCTURE ONLY (see the package docstring).

"Riassunto Tecnico: MatrixFSDP", Metodologia, the MatrixShard metadata and global
planner item: a global planner assigns the owner of every whole matrix so as to
balance the resident bytes and the optimizer work across the ranks.  The page names
no algorithm.  The reading taken: the work of a matrix is its algorithmic
Newton-Schulz flop count, and owners are assigned by the longest-processing-time
rule (Graham): matrices in decreasing order of work (ties: more bytes first, then the
lower index), each to the rank with the least work so far (ties: the fewest bytes,
then the lowest rank).  Bytes are rows * cols * bytes_per_element.

Pins: optimal_makespan (brute force over every assignment) bounds the rule from
below, and Graham's theorem bounds it from above by (4/3 - 1/(3R)) times the optimum.
"""

import itertools


def ns_work(rows, cols, iters):
    """iters * (m^2 n + m^3 + 2 m^2 n) with m = min, n = max: the upper triangle of
    X X^T, A^2 counted once (symmetric), and B X."""
    m, n = min(rows, cols), max(rows, cols)
    return float(iters) * (m * m * n + m ** 3 + 2 * m * m * n)


def lpt_owners(shapes, ranks, iters, bytes_per_element=4.0):
    """Owner per matrix by the longest-processing-time rule with the stated ties.
    Returns (owners, per-rank work, per-rank bytes)."""
    work = [ns_work(r, c, iters) for r, c in shapes]
    nbytes = [float(r) * float(c) * bytes_per_element for r, c in shapes]
    order = sorted(range(len(shapes)), key=lambda i: (-work[i], -nbytes[i], i))
    load_w = [0.0] * ranks
    load_b = [0.0] * ranks
    owners = [None] * len(shapes)
    for i in order:
        best = min(range(ranks), key=lambda r: (load_w[r], load_b[r], r))
        owners[i] = best
        load_w[best] += work[i]
        load_b[best] += nbytes[i]
    return owners, load_w, load_b


def makespan(owners, works, ranks):
    """The largest per-rank sum of work for an assignment."""
    load = [0.0] * ranks
    for o, w in zip(owners, works):
        load[o] += w
    return max(load) if load else 0.0


def optimal_makespan(works, ranks):
    """Smallest possible makespan, by trying every assignment (tiny inputs only)."""
    best = float("inf")
    for assign in itertools.product(range(ranks), repeat=len(works)):
        best = min(best, makespan(assign, works, ranks))
    return best if works else 0.0
