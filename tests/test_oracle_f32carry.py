"""Pins of the oracle's fp32-carry fold (bf16 data, fp32 partials, one final
rounding): the reading of "fp32 accumulation, bf16 round-to-nearest-even
output" in which the reduce-scatter carries fp32 partials.

Each pin is fixed by something other than the fold itself: hand-derived
values, the per-hop fold where both readings coincide, and a brute-force
integer sum rounded by torch's own bf16 conversion."""
import numpy as np
import pytest
import torch

import oracle

ONE, TWO_M8, TWO_P24, NEG_TWO_P24 = 0x3F80, 0x3B80, 0x4B80, 0xCB80   # 1.0, 2^-8, 2^24, -2^24


def u16(vals):
    return np.array(vals, dtype=np.uint16)


def test_one_rank_is_the_input_bit_for_bit():
    x = u16([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x0001, 0x3F80, 0x4049])
    out = oracle.allreduce_fold_f32carry([x])
    assert np.array_equal(out[0], x)   # NaN payloads survive: nothing is added


def test_two_ranks_equal_the_per_hop_fold():
    # With two ranks there is one add and one rounding in both readings.
    g = np.random.default_rng(11)
    xs = [g.integers(0, 1 << 16, 5000, dtype=np.uint64).astype(np.uint16) for _ in range(2)]
    assert np.array_equal(oracle.allreduce_fold_f32carry(xs)[0], oracle.allreduce_fold(xs)[0])


def test_one_rounding_keeps_what_per_hop_rounding_drops():
    # Slice j of element j (n = R = 4): rank j+1 holds 1.0, the other three
    # hold 2^-8.  fp32 carry: 1 + 3*2^-8 = 1 + 1.5 ulp(bf16), a tie between
    # 1 + 2^-7 and 1 + 2^-6, to even: 1 + 2^-6 = 0x3F82.  Per hop: 1 + 2^-8 is
    # a tie between 1 and 1 + 2^-7, to even: 1.0, three times over.
    R = 4
    xs = [u16([ONE if r == (j + 1) % R else TWO_M8 for j in range(R)]) for r in range(R)]
    carry = oracle.allreduce_fold_f32carry(xs)
    per_hop = oracle.allreduce_fold(xs)
    for r in range(R):
        assert carry[r].tolist() == [0x3F82] * R
        assert per_hop[r].tolist() == [ONE] * R


@pytest.mark.parametrize("pattern, want", [
    # ranks j+1, j+2, j+3, j hold: 2^24, -2^24, 0, 1.  In ring order
    # (2^24 - 2^24) + 0 + 1 = 1.  Started at rank j instead: 1 + 2^24 rounds
    # to 2^24 in fp32 (a tie, to even), so the result would be 0.
    ((TWO_P24, NEG_TWO_P24, 0x0000, ONE), ONE),
    # ranks j+1, j+2, j+3, j hold: 1, 2^24, -2^24, 0.  In ring order
    # 1 + 2^24 = 2^24, then 0.  Taken in reverse ring order: -2^24 + 2^24 + 1 = 1.
    ((ONE, TWO_P24, NEG_TWO_P24, 0x0000), 0x0000),
])
def test_fold_order(pattern, want):
    R = 4
    xs = [u16([pattern[(r - j - 1) % R] for j in range(R)]) for r in range(R)]
    assert oracle.allreduce_fold_f32carry(xs)[0].tolist() == [want] * R


def test_integer_sums_round_once_like_torch():
    # Integers in [-128, 128] are exact in bf16, and every partial of 8 of
    # them is an exact fp32 integer, so the result is the exact sum rounded
    # to bf16 once.  torch's own float32 -> bfloat16 conversion (nearest even)
    # rounds the exact sums.
    R, n = 8, 8 * 37 + 5
    g = np.random.default_rng(5)
    ints = [g.integers(-128, 129, n) for _ in range(R)]
    xs = [torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
          for v in ints]
    exact = np.sum(np.stack(ints), axis=0).astype(np.float32)
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.allreduce_fold_f32carry(xs)
    for r in range(R):
        assert np.array_equal(got[r], want)
    # The per-hop fold rounds partials above 256 and so differs somewhere.
    assert not np.array_equal(oracle.allreduce_fold(xs)[0], want)


def test_nan_and_inf():
    R = 3
    nan, inf, ninf = 0x7FC1, 0x7F80, 0xFF80
    xs = [u16([nan, inf, inf, 0x3F80]), u16([0x3F80, ninf, 0x3F80, 0x7F7F]), u16([0x3F80, 0x3F80, inf, 0x7F7F])]
    out = oracle.allreduce_fold_f32carry(xs)[0].tolist()
    assert out[0] == 0x7FC0              # NaN in: canonical NaN out
    assert out[1] == 0x7FC0              # inf + -inf
    assert out[2] == inf
    # 0x7F7F is the largest finite bf16 (about 3.39e38): two of them overflow
    # fp32 (largest finite about 3.40e38) to inf before the final rounding.
    assert out[3] == inf
