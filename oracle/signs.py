"""Oracle for the Sign-Muon tail: elementwise sign, 1-bit packing, majority vote.
TEST INFRASTRUCTURE ONLY (see the package docstring).

"Riepilogo Tecnico: SignMuon", section 2:
  * core mechanism item 2 and distributed flow item 2: each worker keeps only the
    elementwise signs S = sign(U), valued in {-1, +1};
  * distributed flow item 3 and "Efficienza di Comunicazione": signs travel packed
    at one bit per element (32x less than float32), or as int8;
  * core mechanism item 3 and flow item 4: the vote is the integer sum of the
    workers' signs followed by a local threshold sign(sum_m S^(m)).

Readings of what the pages leave open:
  * the sign of 0 and -0 is +1 (bit 1); NaN gives -1 (bit 0, outside the contract);
  * bit layout: flat row-major element i lives in word i // 32 at bit i % 32
    (least significant bit first), bit 1 means +1, unused bits of the last word are 0;
    M workers' packed buffers are stacked as a [M][nwords] array;
  * a tied vote (sum 0, possible for even M) resolves to +1;
  * the integer sum is 2*count - M, which fits int8 for M <= 127;
  * flow item 4 updates the weight with the voted signs, W <- W - eta * S; the
    difference is formed in float32 and stored in the weight's dtype (float32, or
    bfloat16 rounded to nearest even from that float32 value);
  * flow item 5's optional local polar step takes the voted signs as +1 / -1
    values.
"""

import numpy as np


def sign_bits(u):
    """1 where u >= 0 (so +0 and -0 map to +1), else 0; NaN compares false -> 0."""
    return (np.asarray(u).reshape(-1) >= 0).astype(np.uint8)


def pack_bits(bits):
    """Pack a flat 0/1 array LSB-first into ceil(numel/32) uint32 words."""
    bits = np.asarray(bits, dtype=np.uint64).reshape(-1)
    numel = bits.size
    nwords = (numel + 31) // 32
    padded = np.zeros(nwords * 32, dtype=np.uint64)
    padded[:numel] = bits
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    words = (padded.reshape(nwords, 32) * weights).sum(axis=1)
    return words.astype(np.uint32)


def unpack_bits(words, numel):
    """Inverse of pack_bits: the first numel bits as a 0/1 uint8 array."""
    w = np.asarray(words, dtype=np.uint32).reshape(-1).astype(np.uint64)
    shifts = np.arange(32, dtype=np.uint64)
    bits = ((w[:, None] >> shifts[None, :]) & np.uint64(1)).reshape(-1)
    return bits[:numel].astype(np.uint8)


def sign_pack(u):
    """sign then pack, over the flat row-major order of u."""
    return pack_bits(sign_bits(u))


def majority_vote(packed, numel):
    """Majority vote over M packed sign buffers ([M][nwords] uint32).

    Returns (out_words, sums): out bit i is 1 iff sum_i >= 0, where
    sum_i = sum over workers of (+1 if bit else -1) = 2*count_i - M.
    sums is int64 of length numel.
    """
    packed = np.asarray(packed, dtype=np.uint32)
    if packed.ndim != 2:
        raise ValueError("packed must be [M][nwords]")
    M = packed.shape[0]
    counts = np.zeros(numel, dtype=np.int64)
    for w in range(M):
        counts += unpack_bits(packed[w], numel)
    sums = 2 * counts - M
    return pack_bits((sums >= 0).astype(np.uint8)), sums


def unpack_signs(words, numel):
    """The voted sign matrix as values: +1.0 where the bit is set, -1.0 elsewhere
    (float64, flat order).  Input of the optional local polar step (flow item 5)."""
    return np.where(unpack_bits(words, numel) == 1, 1.0, -1.0)


def _round_bf16(x32):
    """float32 -> nearest bfloat16 value, ties to the even one, returned as float64.

    Written from the definition: the two bfloat16 neighbours of x are the values whose
    low 16 bits of the float32 pattern are zero below and above x; pick the nearer,
    on a tie the one whose last kept bit is 0.  Finite inputs only."""
    x = np.asarray(x32, dtype=np.float32).reshape(-1)
    bits = x.view(np.uint32).astype(np.uint64)
    down = bits & np.uint64(0xFFFF0000)            # truncation towards zero
    up = down + np.uint64(0x10000)                 # next value away from zero
    lo = down.astype(np.uint32).view(np.float32).astype(np.float64)
    hi = up.astype(np.uint32).view(np.float32).astype(np.float64)
    xv = x.astype(np.float64)
    d_lo, d_hi = np.abs(xv - lo), np.abs(hi - xv)
    even_lo = ((down >> np.uint64(16)) & np.uint64(1)) == 0
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & even_lo)
    return np.where(take_lo, lo, hi)


def sign_update(weight, words, lr, bf16=False):
    """W - lr * S for the voted signs S (flow item 4), as stored.

    weight: float32 values (for bf16 weights, the float32 values of the bf16 numbers);
    the difference is one float32 subtraction (numpy's float32 arithmetic is IEEE
    correctly rounded), then rounded to bfloat16 when bf16=True.  Returns float64."""
    w = np.asarray(weight, dtype=np.float32).reshape(-1)
    s = unpack_signs(words, w.size).astype(np.float32)
    step = np.float32(lr) * s                      # exact: multiplying by +-1
    diff = (w - step).astype(np.float32)
    return _round_bf16(diff) if bf16 else diff.astype(np.float64)
