"""GPU parity of the one-launch allreduce, in which each workgroup carries one
chunk through every hop of the ring ("ResCCL: Resource-Efficient Scheduling
for Collective Communication", section 3: dependencies exist only within a
chunk, and a generated kernel loops over its work inside the kernel).

HC_CHAIN_MAX_BYTES decides which allreduces take it; here it is set so that
every call does (or none does), and each result is compared with the oracle's
fold bit for bit: the hops are the ring's, in the ring's order."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import bits, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 8, 1000, 4096 * 3 + 5, 65536, 300_001, 8 * 40000 + 24]


def rand(R, n, dtype, seed, scale=1.0):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * scale).astype(np.float32) for _ in range(R)]
    if dtype == "bf16":
        xs = [inputs.f32_to_bf16_bits(x) for x in xs]
    return xs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 4, 5, 8])
def test_chain_allreduce_matches_oracle(monkeypatch, dtype, R):
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", str(1 << 40))
    for n in SIZES:
        xs = rand(R, n, dtype, 700 * R + n, 1e-3 if dtype == "bf16" else 1.0)
        ref = oracle.allreduce_fold(xs)
        send = [to_dev(x) for x in xs]
        recv = [torch.empty_like(t) for t in send]
        hc.hc_allreduce(send, recv)
        hc.hc_allreduce(send, send)          # in place
        torch.cuda.synchronize()
        for r in range(R):
            want = bits(ref[r])
            assert np.array_equal(to_host(recv[r]), want), f"n={n} rank={r}: {first_mismatch(to_host(recv[r]), want)}"
            assert np.array_equal(to_host(send[r]), want), f"in place n={n} rank={r}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_allreduce_options(monkeypatch, dtype):
    """Chunk fractions from one tile to the whole slice, CU budgets (a
    persistent grid over the chunks), and offset views that force the
    element path: the values never change."""
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", str(1 << 40))
    R, n = 8, 8 * 40000 + 24
    xs = rand(R, n, dtype, 11, 1e-2)
    ref = oracle.allreduce_fold(xs)
    for kw in ({}, {"chunk_fraction": 0.001}, {"chunk_fraction": 0.3}, {"chunk_fraction": 1.0},
               {"cu_budget": 1}, {"cu_budget": 8}):
        send = [to_dev(x) for x in xs]
        recv = [torch.empty_like(t) for t in send]
        hc.hc_allreduce(send, recv, **kw)
        torch.cuda.synchronize()
        for r in range(R):
            assert np.array_equal(to_host(recv[r]), bits(ref[r])), f"{kw} rank={r}"
    # buffers that start 2 elements into an allocation: the element path
    big = [to_dev(np.concatenate([np.zeros(2, dtype=x.dtype), x])) for x in xs]
    out = [torch.empty_like(t) for t in big]
    hc.hc_allreduce([t[2:] for t in big], [o[2:] for o in out], n)
    torch.cuda.synchronize()
    for r in range(R):
        assert np.array_equal(to_host(out[r][2:]), bits(ref[r])), f"offset views rank={r}"


def test_chain_and_step_schedules_agree(monkeypatch):
    """The same allreduce through both schedules gives the same bits."""
    R, n = 8, 1 << 20
    xs = rand(R, n, "bf16", 12, 1e-3)
    send = [to_dev(x) for x in xs]
    a = [torch.empty_like(t) for t in send]
    b = [torch.empty_like(t) for t in send]
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", str(1 << 40))
    hc.hc_allreduce(send, a)
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", "0")
    hc.hc_allreduce(send, b)
    torch.cuda.synchronize()
    ref = oracle.allreduce_fold(xs)
    for r in range(R):
        assert np.array_equal(to_host(a[r]), ref[r]) and np.array_equal(to_host(b[r]), ref[r])
