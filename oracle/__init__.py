"""Plain, slow, fp64 CPU oracle for the owner-local Muon step and the Sign-Muon tail.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call or link this package; only the tests, the smoke
check and the CPU-baseline leg of the benchmark use it.  It shares no code with the
GPU path: no kernels, headers, helpers or constant tables.

Sources (web pages, cited by title and section):
  * "Riassunto Tecnico: MatrixFSDP" (gist.science, paper 2607.05895), section
    "Metodologia: MatrixFSDP", item 1 (owner-shaped placement): each owner rank holds
    whole 2D matrices and runs the Newton-Schulz update on them locally.
  * "Riepilogo Tecnico: SignMuon", section 2 "Metodologia: Sign-Muon" (core
    mechanism items 1-3 and the distributed flow items 1-4), section 2 "Efficienza di
    Comunicazione", section 3 (update spectral norm at most 1) and section 4
    (nanoGPT: Frobenius scaling, often one NS iteration).
  The quintic form X <- aX + (bA + cA^2)X with A = X X^T, the heavy-ball momentum,
  the epsilon, the orientation rule and the bit layout are readings of points the
  pages leave open; each function states the reading it takes.

Pins (what ties these functions to something other than themselves) live in
tests/test_oracle_*.py: the singular-value closed form of the iteration, the SVD
polar factor for convergent coefficients, orthogonal equivariance, exact rational
arithmetic for the fused momentum rounding, and brute-force bit counts.
"""

from .muon import (  # noqa: F401
    momentum_update,
    momentum_state_fp32,
    frobenius_normalize,
    newton_schulz,
    ns_orthogonalize,
    muon_step,
    weight_update,
    ns_polynomial_flops,
)
from .signs import (  # noqa: F401
    sign_bits,
    pack_bits,
    unpack_bits,
    sign_pack,
    majority_vote,
    unpack_signs,
    sign_update,
)
from .planner import (  # noqa: F401
    ns_work,
    lpt_owners,
    makespan,
    optimal_makespan,
)
