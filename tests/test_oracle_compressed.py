"""Pins of the oracle's compressed ring allreduce and the contention rate.

Compressed ring: "CCCL: In-GPU Compression-Coupled Collective Communication",
section 5 ("Selective compression": compress what a rank sends, decompress what
it receives, reduce in between) on the ring of "ResCCL: Resource-Efficient
Scheduling for Collective Communication" section 1.  Contention rate: "HOCCL:
Offloading Collective Communication from GPU Cores to Accelerate Distributed
Training", section 2 (formula lost; reading in oracle/hc_oracle.c)."""
import numpy as np
import pytest
import torch

import oracle

B = 16384


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("R,n,chunk", [(2, 2 * B, B), (3, 3 * B + 300, B), (4, 8 * B, 2 * B), (8, 16 * B, B),
                                       (1, 100, B), (5, 7, B)])
def test_compressed_equals_uncompressed(R, n, chunk):
    g = np.random.default_rng(R * 1000 + n)
    xs = [bf16(g.standard_normal(n) * 1e-3) for _ in range(R)]
    outs, wire = oracle.compressed_allreduce(xs, chunk=chunk)
    ref = oracle.allreduce_fold(xs)
    for r in range(R):
        np.testing.assert_array_equal(outs[r], ref[r])
    if R > 1:
        raw = 2 * (R - 1) * R * oracle.slice_len(n, R) * 2
        assert wire > 0
        if n >= R * B:
            assert wire < raw          # compression pays on gradient-like data


def test_wire_bytes_hand_derived():
    """R=2, two ranks of 2*16384 elements all 1.0, chunk = one block.  Each
    slice is one block.  Reduce-scatter: each sender ships its input slice
    (constant 1.0 -> one coded block, b=1, 18464 B; stream 48 + 18464 = 18512).
    All-gather: each receiver gets the finished slice, constant 2.0, again one
    18512-byte stream.  Two RS streams + two AG streams = 4 * 18512 = 74048."""
    xs = [np.full(2 * B, 0x3F80, np.uint16) for _ in range(2)]
    outs, wire = oracle.compressed_allreduce(xs, chunk=B)
    assert wire == 4 * 18512
    for o in outs:
        assert np.all(o == 0x4000)


def test_wire_bytes_count_raw_tail_blocks():
    """R=2, slice = 16384 + 8: each slice ships as one stream with a coded block
    (18464) and a raw 8-element tail (16 + 16 = 32); stream = 32 + 16 + 18464 + 32
    = 18544 bytes; four streams."""
    n = 2 * (B + 8)
    xs = [np.full(n, 0x3F80, np.uint16) for _ in range(2)]
    _, wire = oracle.compressed_allreduce(xs, chunk=2 * B)
    assert wire == 4 * 18544


def test_contention_rate_hand_intervals():
    # compute over [0, 10]; a 32-CU reduce over [2, 7] on a 256-CU part:
    # (5 * 32/256) / 10 = 0.0625
    assert oracle.contention_rate([(0, 10)], [(2, 7, 32)], 256) == pytest.approx(0.0625)
    # compute [0,4] and [6,10]; 16 CUs over [3,8]: overlap 1 + 2 = 3 units of 8
    assert oracle.contention_rate([(0, 4), (6, 10)], [(3, 8, 16)], 256) == pytest.approx(3 * 16 / 256 / 8)
    # two traffic intervals overlapping each other add their CUs
    assert oracle.contention_rate([(0, 4)], [(0, 2, 8), (1, 3, 8)], 256) == pytest.approx(
        (1 * 8 + 1 * 16 + 1 * 8) / 256 / 4)
    # the reduce spanning all compute time: exactly k / 256
    for k in (8, 16, 32):
        assert oracle.contention_rate([(1, 2)], [(0, 3, k)], 256) == pytest.approx(k / 256)
    assert oracle.contention_rate([], [(0, 1, 8)], 256) == -1.0
