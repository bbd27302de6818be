"""Seeded synthetic inputs for the owner-local Muon step and the Sign-Muon vote.

This module is the only code the GPU path's callers and the oracle's callers share.
It holds shapes, seeds, distributions and dtype casts of INPUTS; it computes nothing
the method computes.

Workloads (owner sets of whole 2D matrices, listed layer-major in the order given):
  1  single-256x128:   one 256 x 128 fp32 matrix, G and prior M i.i.d. N(0, 1)
  2  125m-class:       12 x {4 x 768x768, 768x3072, 3072x768}; bf16 G ~ N(0, 0.02^2),
                       fp32 prior M from the same distribution
  3  1b-class-swiglu:  16 x {4 x 2048x2048, 2 x 2048x5632, 5632x2048}; bf16 G ~
                       N(0, 0.01^2) with round(1% of rows) scaled by 10 before the
                       bf16 cast (heavy-tailed), fp32 prior M ~ N(0, 0.01^2)
  4  7b-class:         32 x {4 x 4096x4096, 2 x 4096x11008, 11008x4096}; bf16 G ~
                       N(0, 0.01^2), fp32 prior M ~ N(0, 0.01^2)
  5  sign-vote-8x4096: 8 workers, each a 4096x4096 fp32 momentum ~ N(0, 1) with
                       its own seed (the momentum is given; no momentum update)

Host generator (numpy, used wherever the oracle checks a result):
  default_rng([workload, matrix_index, tensor_id]) with tensor_id 0 = gradient,
  1 = prior momentum, 2 = heavy-tail row choice; float32 normals times a float32
  sigma (one rounding), then round-to-nearest-even to bf16 where the gradient is
  bf16.  Workload 5 uses [5, worker, 1].

Device generator (torch, for the bulk of full-size runs whose outputs are not
checked one by one): the same distributions from torch.Generator seeded with
1_000_003 * workload + matrix_index, so a full 7B-class owner set materialises in
milliseconds instead of minutes of host RNG.
"""

from dataclasses import dataclass
import numpy as np

# Commonly published aggressive quintic Muon coefficients.  They are NOT on the
# pages (which print no coefficients); they are a caller-chosen default.
MUON_ABC = (3.4445, -4.7750, 2.0315)
# Convergent "textbook" quintic: Taylor polynomial of (1 - z)^(-1/2) at z = 1 - s^2.
TEXTBOOK_QUINTIC_ABC = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)
TEXTBOOK_CUBIC_ABC = (1.5, -0.5, 0.0)
BETA = 0.95
EPS = 1e-7


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    layer_shapes: tuple          # shapes of one layer, in listing order
    layers: int
    grad_dtype: str              # "f32" | "bf16"
    grad_std: float
    mom_std: float
    compute: str                 # "f32" | "bf16"
    iters: int = 5
    heavy_tail: bool = False

    @property
    def shapes(self):
        return [s for _ in range(self.layers) for s in self.layer_shapes]

    @property
    def count(self):
        return self.layers * len(self.layer_shapes)

    @property
    def numel(self):
        return sum(r * c for r, c in self.shapes)


WORKLOADS = {
    1: Workload(1, "single-256x128", ((256, 128),), 1, "f32", 1.0, 1.0, "f32"),
    2: Workload(2, "125m-class", ((768, 768),) * 4 + ((768, 3072), (3072, 768)), 12,
                "bf16", 0.02, 0.02, "bf16"),
    3: Workload(3, "1b-class-swiglu", ((2048, 2048),) * 4 + ((2048, 5632),) * 2 + ((5632, 2048),),
                16, "bf16", 0.01, 0.01, "bf16", heavy_tail=True),
    4: Workload(4, "7b-class", ((4096, 4096),) * 4 + ((4096, 11008),) * 2 + ((11008, 4096),), 32,
                "bf16", 0.01, 0.01, "bf16"),
    5: Workload(5, "sign-vote-8x4096", ((4096, 4096),), 8, "f32", 1.0, 1.0, "bf16"),
}


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normals(seed, shape, std):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def heavy_tail_rows(wid, idx, rows):
    """round(1% of rows) distinct row indices, from a seeded permutation."""
    k = int(round(0.01 * rows))
    return np.sort(np.random.default_rng([wid, idx, 2]).permutation(rows)[:k])


def host_matrix(wid, idx):
    """Inputs of matrix idx of workload wid, on the host.

    Returns dict(grad=float32 exact values, grad_bits=uint16 or None,
    mom=float32 prior momentum, shape=(r, s)).
    """
    w = WORKLOADS[wid]
    r, s = w.shapes[idx]
    if wid == 5:
        mom = _normals([5, idx, 1], (r, s), w.mom_std)
        return dict(grad=None, grad_bits=None, mom=mom, shape=(r, s))
    g = _normals([wid, idx, 0], (r, s), w.grad_std)
    if w.heavy_tail:
        g[heavy_tail_rows(wid, idx, r)] *= np.float32(10.0)
    bits = None
    if w.grad_dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        g = bf16_bits_to_f32(bits)
    mom = _normals([wid, idx, 1], (r, s), w.mom_std)
    return dict(grad=g, grad_bits=bits, mom=mom, shape=(r, s))


def device_seed(wid, idx):
    return 1_000_003 * wid + idx


def device_matrix(wid, idx, device):
    """Same distributions as host_matrix, drawn by torch's generator on `device`.
    Returns (grad tensor in the workload's grad dtype or None, fp32 momentum)."""
    import torch
    w = WORKLOADS[wid]
    r, s = w.shapes[idx]
    gen = torch.Generator(device=device)
    gen.manual_seed(device_seed(wid, idx))
    mom = torch.randn(r, s, generator=gen, device=device, dtype=torch.float32) * w.mom_std
    if wid == 5:
        return None, mom
    g = torch.randn(r, s, generator=gen, device=device, dtype=torch.float32) * w.grad_std
    if w.heavy_tail:
        rows = torch.randperm(r, generator=gen, device=device)[: int(round(0.01 * r))]
        g[rows] *= 10.0
    if w.grad_dtype == "bf16":
        g = g.to(torch.bfloat16)
    return g, mom
