"""Pins of the sign / 1-bit pack / majority-vote oracle against hand-derived cases,
brute force and invariants (CPU only).  The pages print no worked numeric example,
so the hand cases below are derived from the definitions: bit = 1 iff u >= 0,
element i at bit i % 32 of word i // 32, vote = sign of the integer sum, tie -> +1."""

import numpy as np
import pytest

import oracle
from pins import brute_pack, brute_vote


def test_hand_derived_pack_cases():
    # +1, -1, +0, -0 -> bits 1, 0, 1, 1 -> 0b1101
    assert oracle.sign_pack(np.array([1.0, -1.0, 0.0, -0.0])).tolist() == [0xD]
    # 31 negatives then one non-negative -> only the top bit
    v = -np.ones(32)
    v[31] = 0.5
    assert oracle.sign_pack(v).tolist() == [0x80000000]
    # 33 positives -> a full word and one bit of the next, pad bits zero
    assert oracle.sign_pack(np.ones(33)).tolist() == [0xFFFFFFFF, 0x1]
    # NaN is outside the contract and maps to bit 0
    assert oracle.sign_pack(np.array([np.nan, 1.0])).tolist() == [0x2]
    # 1-bit payload: ceil(numel / 32) words, i.e. numel / 8 bytes
    assert oracle.sign_pack(np.zeros(4096 * 4096, np.float32)).nbytes == 4096 * 4096 // 8


def test_hand_derived_vote_cases():
    out, sums = oracle.majority_vote(np.array([[0b011], [0b101], [0b110]], np.uint32), 3)
    assert out.tolist() == [0b111] and sums.tolist() == [1, 1, 1]
    out, sums = oracle.majority_vote(np.array([[0b01], [0b10]], np.uint32), 2)
    assert out.tolist() == [0b11] and sums.tolist() == [0, 0]      # ties -> +1
    out, sums = oracle.majority_vote(np.array([[0b00], [0b01]], np.uint32), 2)
    assert out.tolist() == [0b01] and sums.tolist() == [0, -2]
    out, sums = oracle.majority_vote(np.array([[0b1]], np.uint32), 1)
    assert out.tolist() == [0b1] and sums.tolist() == [1]


@pytest.mark.parametrize("numel", [1, 5, 31, 32, 33, 63, 64, 65, 100, 200])
def test_pack_matches_brute_force(numel):
    rng = np.random.default_rng(numel)
    v = rng.standard_normal(numel)
    v[rng.random(numel) < 0.1] = 0.0
    v[rng.random(numel) < 0.1] = -0.0
    np.testing.assert_array_equal(oracle.sign_pack(v), brute_pack(v))
    np.testing.assert_array_equal(oracle.unpack_bits(oracle.sign_pack(v), numel),
                                  (v >= 0).astype(np.uint8))


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 9])
@pytest.mark.parametrize("numel", [1, 31, 32, 33, 64, 97, 200])
def test_vote_matches_brute_force(M, numel):
    rng = np.random.default_rng(M * 1000 + numel)
    packed = np.stack([oracle.sign_pack(rng.standard_normal(numel)) for _ in range(M)])
    out, sums = oracle.majority_vote(packed, numel)
    want_out, want_sums = brute_vote(list(packed), numel)
    np.testing.assert_array_equal(out, want_out)
    np.testing.assert_array_equal(sums, want_sums)


def test_vote_invariants():
    rng = np.random.default_rng(3)
    numel = 1000
    s = oracle.sign_pack(rng.standard_normal(numel))
    # M = 1 is the identity
    out, _ = oracle.majority_vote(s[None], numel)
    np.testing.assert_array_equal(out, s)
    # (S, -S): every element ties -> all +1, pad bits stay 0
    neg = oracle.pack_bits(1 - oracle.unpack_bits(s, numel))
    out, sums = oracle.majority_vote(np.stack([s, neg]), numel)
    assert np.all(sums == 0)
    np.testing.assert_array_equal(out, oracle.pack_bits(np.ones(numel)))
    # order of workers does not matter
    p = np.stack([oracle.sign_pack(rng.standard_normal(numel)) for _ in range(5)])
    a, _ = oracle.majority_vote(p, numel)
    b, _ = oracle.majority_vote(p[::-1], numel)
    np.testing.assert_array_equal(a, b)
    # odd M: negating every input negates the output (no ties possible)
    pn = np.stack([oracle.pack_bits(1 - oracle.unpack_bits(r, numel)) for r in p])
    c, _ = oracle.majority_vote(pn, numel)
    np.testing.assert_array_equal(oracle.unpack_bits(c, numel), 1 - oracle.unpack_bits(a, numel))


# ------------------------------------------------ voted-sign unpack and update

@pytest.mark.parametrize("numel", [1, 5, 31, 32, 33, 95, 200])
def test_unpack_signs_brute_force(numel):
    rng = np.random.default_rng(numel)
    words = rng.integers(0, 2 ** 32, (numel + 31) // 32, dtype=np.uint64).astype(np.uint32)
    want = []
    for i in range(numel):
        bit = (int(words[i // 32]) >> (i % 32)) & 1
        want.append(1.0 if bit else -1.0)
    np.testing.assert_array_equal(oracle.unpack_signs(words, numel), np.array(want))


def test_round_bf16_matches_torch_cpu_conversion():
    import torch
    from oracle.signs import _round_bf16
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 6, 20000)).astype(np.float32)
    ties = (np.arange(1, 300, dtype=np.uint32) << 16 | 0x8000).view(np.float32)   # exact halfway points
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0, -1.5])])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(_round_bf16(x), want)


def test_sign_update_hand_cases():
    words = np.array([0b0101], dtype=np.uint32)            # signs +1, -1, +1, -1
    w = np.float32([1.0, 1.0, -2.0, 0.25])
    got = oracle.sign_update(w, words, 0.5)
    np.testing.assert_array_equal(got, [0.5, 1.5, -2.5, 0.75])
    # bf16: 1 - 2^-9 lies exactly halfway between the bf16 numbers 1 - 2^-8 and 1;
    # the even one is 1.0 (mantissa ...0)
    got = oracle.sign_update(np.float32([1.0]), np.array([1], np.uint32), 2.0 ** -9, bf16=True)
    np.testing.assert_array_equal(got, [1.0])
    # float32 rounding: 1 + 2^-30 is not a float32 and rounds back to 1
    got = oracle.sign_update(np.float32([1.0]), np.array([0], np.uint32), 2.0 ** -30)
    np.testing.assert_array_equal(got, [1.0])
