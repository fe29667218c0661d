"""Pins of the oracle's HCZ1 codec.

Principle from "CCCL: In-GPU Compression-Coupled Collective Communication":
section 4.1 (exponent coded, sign and fraction raw), 4.3 (a local table per
block, fixed-length codes), section 5 "Handling data alignment" (unaligned
remainder sent raw).  Pins: hand-derived worked examples of sizes, plans and
byte layout (tests/golden/codec_examples.txt), all 65,536 bf16 bit patterns
round-trip through raw and coded blocks, the size bound, determinism and the
rejection of corrupted streams."""
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
B = 16384


def build_case(kind: str, args):
    if kind == "fill":
        return np.full(int(args[1]), int(args[0], 16), dtype=np.uint16)
    if kind == "halves":
        return np.concatenate([np.full(B // 2, int(args[0], 16), np.uint16),
                               np.full(B // 2, int(args[1], 16), np.uint16)])
    if kind == "eighth":
        v = np.full(B, int(args[0], 16), np.uint16)
        v[::8] = int(args[1], 16)
        return v
    if kind == "flat256":
        return ((np.arange(B) % 256).astype(np.uint16) << 7).astype(np.uint16)
    raise KeyError(kind)


def read_examples():
    rows = []
    with open(os.path.join(GOLDEN, "codec_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, cons, plan, total = [p.strip() for p in line.split("|")]
            parts = cons.split()
            mode, b, n_esc, rec = (int(v) for v in plan.split())
            rows.append((name, build_case(parts[0], parts[1:]), (mode, b, n_esc, rec), int(total)))
    return rows


@pytest.mark.parametrize("ex", read_examples(), ids=lambda e: e[0])
def test_worked_examples(ex):
    name, v, (mode, b, n_esc, rec), total = ex
    last = v[(len(v) - 1) // B * B:]
    plan = oracle.plan_block(last)
    assert (plan["mode"], plan["b"], plan["n_esc"], plan["rec_bytes"]) == (mode, b, n_esc, rec)
    s = oracle.compress(v)
    assert len(s) == total
    rc, back = oracle.decompress(s, len(v))
    assert rc == oracle.OK
    np.testing.assert_array_equal(back, v)


def test_header_fields():
    v = np.full(B + 5, 0x3F80, np.uint16)
    s = oracle.compress(v)
    magic, blk, n, nb, flags, total = struct.unpack_from("<IIQIIQ", s, 0)
    assert (magic, blk, n, nb, flags, total) == (0x315A4348, B, B + 5, 2, 0, len(s))
    off0, off1 = struct.unpack_from("<QQ", s, 32)
    assert off0 == 48 and off1 == 48 + 18464
    # record header of the coded block: mode 1, b 1, reserved 0, m, n_esc, rec_bytes
    assert struct.unpack_from("<BBHIII", s, off0) == (1, 1, 0, B, 0, 18464)
    # the raw tail record: mode 0, 5 elements, 32 bytes, words then zero padding
    assert struct.unpack_from("<BBHIII", s, off1) == (0, 0, 0, 5, 0, 32)
    assert struct.unpack_from("<5H", s, off1 + 16) == (0x3F80,) * 5
    assert s[off1 + 26:off1 + 32] == bytes(6)


def test_layout_two_halves():
    """Ties in count rank by exponent ascending: 127 gets code 0, 128 code 1.
    Plane 0 holds bit 0 of each code, element i at bit i%8 of byte i/8."""
    v = build_case("halves", ["0x3F80", "0x4000"])
    s = oracle.compress(v)
    r = 48
    body = s[r + 16:]
    dict_bytes = body[:16]
    # dictionary: K = 3 most frequent (127, 128, then the smallest zero-count exponent 0)
    assert dict_bytes == bytes([127, 128, 0]) + bytes(13)
    plane0 = body[16:16 + 2048]
    plane1 = body[16 + 2048:16 + 4096]
    assert plane0 == bytes(1024) + b"\xff" * 1024
    assert plane1 == bytes(2048)
    sm = body[16 + 4096:16 + 4096 + B]
    assert sm == bytes(B)             # sign 0 and fraction 0 everywhere
    assert len(body) == 16 + 4096 + B


def test_layout_every_eighth_escapes():
    """b=1 wins the size tie with b=2; exponent 128 is escaped, so plane 0 has bit
    0 (element 8k) set in every byte and the escape plane lists 128 in order."""
    v = build_case("eighth", ["0x3F80", "0x4000"])
    s = oracle.compress(v)
    body = s[48 + 16:]
    assert body[:16] == bytes([127]) + bytes(15)
    plane0 = body[16:16 + 2048]
    assert plane0 == b"\x01" * 2048
    esc = body[16 + 2048 + B:]
    assert esc == bytes([128]) * 2048


def test_sign_and_fraction_plane():
    g = np.random.default_rng(3)
    frac = g.integers(0, 128, B).astype(np.uint16)
    sign = g.integers(0, 2, B).astype(np.uint16)
    v = (sign << 15) | (np.uint16(127) << 7) | frac
    s = oracle.compress(v.astype(np.uint16))
    body = s[48 + 16:]
    sm = np.frombuffer(body[16 + 2048:16 + 2048 + B], dtype=np.uint8)
    np.testing.assert_array_equal(sm, ((sign << 7) | frac).astype(np.uint8))


def test_all_bit_patterns_round_trip_raw_and_coded():
    pats = np.arange(1 << 16, dtype=np.uint16)
    # consecutive patterns: 128 exponents x 128 each per block -> coded with b=7
    s = oracle.compress(pats)
    rc, back = oracle.decompress(s, pats.size)
    assert rc == oracle.OK
    np.testing.assert_array_equal(back, pats)
    # interleave each pattern into mostly-1.0 blocks: coded, patterns land as
    # dictionary hits or escapes
    g = np.random.default_rng(5)
    per = 1384
    chunks = []
    for k in range(0, pats.size, per):
        blk = np.full(B, 0x3F80, np.uint16)
        part = pats[k:k + per]
        pos = g.choice(B, part.size, replace=False)
        blk[pos] = part
        chunks.append(blk)
    v = np.concatenate(chunks)
    s = oracle.compress(v)
    plans = [oracle.plan_block(v[i:i + B]) for i in range(0, v.size, B)]
    assert all(p["mode"] == 1 for p in plans)
    rc, back = oracle.decompress(s, v.size)
    assert rc == oracle.OK
    np.testing.assert_array_equal(back, v)
    # a raw block holding every exponent equally, with random sign/fraction
    flat = ((np.arange(B) % 256).astype(np.uint16) << 7) | g.integers(0, 128, B).astype(np.uint16)
    flat |= (g.integers(0, 2, B).astype(np.uint16) << 15)
    assert oracle.plan_block(flat)["mode"] == 0
    rc, back = oracle.decompress(oracle.compress(flat), B)
    assert rc == oracle.OK
    np.testing.assert_array_equal(back, flat)


@pytest.mark.parametrize("n", [0, 1, 5, B - 1, B, B + 1, 3 * B + 77])
def test_round_trip_and_bound_ragged(n):
    g = np.random.default_rng(n)
    x = (g.standard_normal(n) * 1e-3).astype(np.float32)
    import torch
    v = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    s = oracle.compress(v)
    assert len(s) <= oracle.compress_bound(n)
    rc, back = oracle.decompress(s, n)
    assert rc == oracle.OK
    np.testing.assert_array_equal(back, v)
    # bound = every block raw: 2n + header + 16-byte record headers and padding
    nb = -(-n // B)
    assert oracle.compress_bound(n) == 32 + (-(-8 * nb // 16)) * 16 + sum(
        16 + (-(-2 * min(B, n - k * B) // 16)) * 16 for k in range(nb))


def test_deterministic_and_seed_sensitive():
    import torch
    g1 = np.random.default_rng(1).standard_normal(2 * B).astype(np.float32) * 0.02
    g2 = np.random.default_rng(2).standard_normal(2 * B).astype(np.float32) * 0.02
    v1 = torch.from_numpy(g1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    v2 = torch.from_numpy(g2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert oracle.compress(v1) == oracle.compress(v1.copy())
    assert oracle.compress(v1) != oracle.compress(v2)
    # decompress then compress gives the same stream back
    s = oracle.compress(v1)
    rc, back = oracle.decompress(s, v1.size)
    assert oracle.compress(back) == s


def test_ratio_of_gaussian_weights_near_seventy_percent():
    """CCCL section 4.1: exponent coding compresses bf16 to about 70% of raw."""
    import torch
    x = np.random.default_rng(9).standard_normal(16 * B).astype(np.float32) * 0.02
    v = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ratio = len(oracle.compress(v)) / (2 * v.size)
    assert 0.65 < ratio < 0.75


def corrupt_cases(s: bytes):
    b = bytearray(s)
    flipped = bytearray(b)
    flipped[0] ^= 1
    yield "magic", bytes(flipped), len(s)
    yield "truncated", s, len(s) - 16
    rb = bytearray(b)
    rec = 48
    v = struct.unpack_from("<I", rb, rec + 12)[0]
    struct.pack_into("<I", rb, rec + 12, v + 16)
    yield "rec_bytes+16", bytes(rb), len(s)
    rb2 = bytearray(b)
    struct.pack_into("<I", rb2, rec + 12, v - 16)
    yield "rec_bytes-16", bytes(rb2), len(s)
    bb = bytearray(b)
    bb[rec + 1] = 9
    yield "b=9", bytes(bb), len(s)
    ne = bytearray(b)
    struct.pack_into("<I", ne, rec + 8, struct.unpack_from("<I", ne, rec + 8)[0] + 1)
    yield "n_esc+1", bytes(ne), len(s)
    off = bytearray(b)
    struct.pack_into("<Q", off, 32, 1 << 40)
    yield "offset", bytes(off), len(s)


def test_corrupt_streams_rejected():
    v = build_case("eighth", ["0x3F80", "0x4000"])
    v = np.concatenate([v, v[:100]])
    s = oracle.compress(v)
    for name, bad, nbytes in corrupt_cases(s):
        rc, out = oracle.decompress(bad[:nbytes], v.size)
        assert rc == oracle.CORRUPT, name
        assert not out.any(), name
    rc, _ = oracle.decompress(s, v.size + 1)    # wrong element count
    assert rc == oracle.CORRUPT
