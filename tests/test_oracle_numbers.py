"""Pins of the oracle's scalar rules (bf16 rounding, the fp32 and bf16 hops)
against routes that share nothing with it: PyTorch's fp32->bf16 conversion and
exact fp64 sums.  CPU only."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def torch_bf16(bits_u32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits_u32.view(np.float32).copy())
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def all_rounding_cases() -> np.ndarray:
    """Every bf16 high half combined with the low halves that decide rounding:
    exact, just above, just below the midpoint, the midpoint (tie) and the top."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


def test_f32_to_bf16_matches_torch_on_every_rounding_case():
    bits = all_rounding_cases()
    ours = oracle.f32_to_bf16_array(bits)
    ref = torch_bf16(bits)
    nan = (bits & 0x7FFFFFFF) > 0x7F800000
    # non-NaN: torch's conversion (nearest even) is the independent route
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # NaN: the oracle's stated reading, one canonical quiet NaN (torch keeps payloads)
    # NaN inputs: 254 high halves above 0x7F80/0xFF80 x 8 lows, plus 0x7F80/0xFF80
    # with the 7 nonzero lows
    assert np.all(ours[nan] == 0x7FC0) and nan.sum() == 254 * 8 + 2 * 7


def test_f32_to_bf16_matches_torch_on_random_words():
    g = np.random.default_rng(7)
    bits = g.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    nan = (bits & 0x7FFFFFFF) > 0x7F800000
    ours = oracle.f32_to_bf16_array(bits)
    np.testing.assert_array_equal(ours[~nan], torch_bf16(bits)[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_f32_to_bf16_hand_cases():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    assert oracle.f32_to_bf16(0x3F808000) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 0x3F82
    assert oracle.f32_to_bf16(0x3F818000) == 0x3F82
    # largest finite fp32 rounds past max bf16 to +inf
    assert oracle.f32_to_bf16(0x7F7FFFFF) == 0x7F80
    # max bf16 + half ulp (tie, max bf16 has an odd significand) -> inf
    assert oracle.f32_to_bf16(0x7F7F8000) == 0x7F80
    # just below that tie stays finite
    assert oracle.f32_to_bf16(0x7F7F7FFF) == 0x7F7F
    # subnormals round like any other value; -0 keeps its sign
    assert oracle.f32_to_bf16(0x00008000) == 0x0000
    assert oracle.f32_to_bf16(0x00018000) == 0x0002
    assert oracle.f32_to_bf16(0x80000000) == 0x8000
    assert oracle.f32_to_bf16(0xFFC00001) == 0x7FC0


def fp64_route_bf16_hop(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact sum in fp64, one rounding to fp32, then bf16 by torch.

    The sum of two bf16 values is exact in fp64 when their exponents differ by
    at most 45; beyond that the smaller is below 2^-45 of the larger and the
    fp64 result cannot land on an fp32 tie, so casting to fp32 gives the
    correctly rounded fp32 sum in all cases."""
    fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        s32 = (fa + fb).astype(np.float32)
    out = torch_bf16(s32.view(np.uint32).copy())
    out[np.isnan(s32)] = 0x7FC0      # the stated canonical NaN of a hop
    return out


def test_bf16_hop_all_a_against_sampled_b():
    g = np.random.default_rng(11)
    a_all = np.arange(1 << 16, dtype=np.uint16)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                         0x7F80, 0xFF80, 0x7FC0, 0x3F80, 0xBF80, 0x4B80, 0xCB80], dtype=np.uint16)
    bs = np.concatenate([specials, g.integers(0, 1 << 16, 113).astype(np.uint16)])
    for bv in bs:
        b = np.full(a_all.size, bv, dtype=np.uint16)
        np.testing.assert_array_equal(oracle.hop_bf16_array(a_all, b), fp64_route_bf16_hop(a_all, b),
                                      err_msg=f"b=0x{int(bv):04x}")


def test_bf16_hop_random_pairs():
    g = np.random.default_rng(12)
    a = g.integers(0, 1 << 16, 4_000_000).astype(np.uint16)
    b = g.integers(0, 1 << 16, 4_000_000).astype(np.uint16)
    np.testing.assert_array_equal(oracle.hop_bf16_array(a, b), fp64_route_bf16_hop(a, b))


def test_f32_hop_against_fp64_route():
    g = np.random.default_rng(13)
    a = g.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    b = g.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    # narrow exponent gaps too, where cancellation and ties happen
    a2 = (g.standard_normal(2_000_000).astype(np.float32)).view(np.uint32)
    b2 = (g.standard_normal(2_000_000).astype(np.float32)).view(np.uint32)
    a = np.concatenate([a, a2])
    b = np.concatenate([b, b2])
    ours = oracle.hop_f32_array(a, b)
    fa = a.view(np.float32).astype(np.float64)
    fb = b.view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = (fa + fb).astype(np.float32)
    ref_bits = ref.view(np.uint32).copy()
    ref_bits[np.isnan(ref)] = 0x7FC00000
    # fp64 sum of two fp32 values is exact when the exponent gap is <= 29 and
    # otherwise cannot create an fp32 tie, so one cast is the correctly rounded sum.
    np.testing.assert_array_equal(ours, ref_bits)


def test_f32_hop_keeps_subnormals_and_signed_zero():
    tiny = 0x00000001  # smallest subnormal
    assert oracle.hop_f32(tiny, tiny) == 0x00000002
    assert oracle.hop_f32(0x80000000, 0x00000000) == 0x00000000  # -0 + +0 = +0
    assert oracle.hop_f32(0x80000000, 0x80000000) == 0x80000000  # -0 + -0 = -0
    assert oracle.hop_f32(0x7F800000, 0xFF800000) == 0x7FC00000  # inf - inf -> canonical NaN


@pytest.mark.parametrize("a,b,expect", [
    (0x3F80, 0x3F80, 0x4000),   # 1 + 1 = 2
    (0x4380, 0x3F80, 0x4380),   # 256 + 1 = 257 -> tie -> 256
    (0x4381, 0x3F80, 0x4382),   # 258 + 1 = 259 -> tie -> 260 (even)
    (0x7F7F, 0x7F7F, 0x7F80),   # overflow to inf
    (0x7F80, 0xFF80, 0x7FC0),   # inf + -inf -> canonical NaN
])
def test_bf16_hop_hand_cases(a, b, expect):
    assert oracle.hop_bf16(a, b) == expect


@pytest.mark.slow
def test_bf16_hop_exhaustive_all_pairs(tmp_path):
    """All 2^32 bf16 (a, b) pairs against an fp64 -> fp32 -> integer-carry
    route (tests/pins/hop_bf16_exhaustive.c), on 8 threads."""
    oracle.lib()  # builds liboracle_hc.so if needed
    so_dir = os.path.dirname(oracle._LIB_PATH)
    exe = tmp_path / "hop_bf16_exhaustive"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-pthread",
                    os.path.join(HERE, "pins", "hop_bf16_exhaustive.c"), "-o", str(exe),
                    f"-L{so_dir}", "-loracle_hc", f"-Wl,-rpath,{so_dir}", "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches=0" in r.stdout
