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
  * the integer sum is 2*count - M, which fits int8 for M <= 127.
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
