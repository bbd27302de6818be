"""Helpers for GPU parity tests: device upload of the seeded inputs, runs through the
binding (C ABI), and error measures."""

import sys

import numpy as np

from matrix_optimizers_sharded_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev_f32(x, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def to_dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)


def host_f32(t):
    """Exact float32 values of a device tensor (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float32)


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    if den == 0:
        return float(np.linalg.norm(got))
    return float(np.linalg.norm(got - want) / den)


def gaussian(shape, seed, std=1.0):
    return (np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std))


def bf16_round(x):
    bits = f32_to_bf16_bits(x)
    return bits, bf16_bits_to_f32(bits)


def run_muon(dev, grads_np, moms_np, grad_dtype, compute, out_dtype, beta, abc, iters, eps, workspace=None):
    """grads_np: float32 arrays (exact values; bf16-representable when grad_dtype is
    bf16).  Returns (new momenta as float32 arrays, U as float32 arrays)."""
    import torch
    from matrix_optimizers_sharded_amd import muon_step_batched
    if grad_dtype == torch.bfloat16:
        grads = [to_dev_bf16(f32_to_bf16_bits(g), dev) for g in grads_np]
    else:
        grads = [to_dev_f32(g, dev) for g in grads_np]
    moms = [to_dev_f32(m, dev) for m in moms_np]
    outs = [torch.empty(g.shape, dtype=out_dtype, device=dev) for g in grads_np]
    muon_step_batched(grads, moms, outs, beta, *abc, iters, eps, compute=compute, workspace=workspace)
    torch.cuda.synchronize()
    return [host_f32(m) for m in moms], [host_f32(o) for o in outs]


def run_ns(dev, xs_np, in_dtype, compute, out_dtype, abc, iters, eps):
    import torch
    from matrix_optimizers_sharded_amd import ns_orthogonalize
    if in_dtype == torch.bfloat16:
        xs = [to_dev_bf16(f32_to_bf16_bits(x), dev) for x in xs_np]
    else:
        xs = [to_dev_f32(x, dev) for x in xs_np]
    outs = [torch.empty(x.shape, dtype=out_dtype, device=dev) for x in xs_np]
    ns_orthogonalize(xs, outs, *abc, iters, eps, compute=compute)
    torch.cuda.synchronize()
    return [host_f32(o) for o in outs]
