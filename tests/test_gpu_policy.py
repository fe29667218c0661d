"""GPU parity of the ring hops under each launch policy.

A step launch moves its tiles one of three ways: 2 vectors per lane and
ordinary stores (the default), 1 vector per lane and non-temporal stores
(launches that write at least HC_STREAM_STORE_MIN_BYTES, 320 MiB by
default), or 4 vectors per lane on a CU budget.  The values must not depend
on it.  Here the environment threshold is set to 0 (or 1) so that every
launch of small, ragged shapes takes the streaming policy, and each result
is compared with the oracle bit for bit; the budget policy is run the same
way with cu_budget.  Source of the operations: "ResCCL: Resource-Efficient
Scheduling for Collective Communication" (section 1, recvReduceCopy and copy
hops) and "Breaking the computation and communication abstraction barrier in
distributed machine learning workloads" ("The idea": AllReduce =
ReduceScatter + AllGather, the update between them)."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import bits, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu

SIZES = [1, 7, 1000, 8192 * 3 + 17, 65536, 300_001, 8 * 40000 + 24]


def rand(R, n, dtype, seed, scale=1.0):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * scale).astype(np.float32) for _ in range(R)]
    if dtype == "bf16":
        xs = [inputs.f32_to_bf16_bits(x) for x in xs]
    return xs


POLICIES = [({"HC_STREAM_STORE_MIN_BYTES": "0"}, {}), ({"HC_STREAM_STORE_MIN_BYTES": "1"}, {}),
            ({}, {"cu_budget": 3}), ({}, {"cu_budget": 64})]
IDS = ["stream0", "stream1", "budget3", "budget64"]


@pytest.mark.parametrize("env,kw", POLICIES, ids=IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_allreduce_each_policy(monkeypatch, env, kw, dtype, R):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    for n in SIZES:
        xs = rand(R, n, dtype, 500 * R + n, 1e-3 if dtype == "bf16" else 1.0)
        ref = oracle.allreduce_fold(xs)
        send = [to_dev(x) for x in xs]
        recv = [torch.empty_like(s) for s in send]
        hc.hc_allreduce(send, recv, **kw)
        hc.hc_allreduce(send, send, **kw)        # in place
        torch.cuda.synchronize()
        for r in range(R):
            want = bits(ref[r])
            got = to_host(recv[r])
            assert np.array_equal(got, want), f"n={n} rank={r}: {first_mismatch(got, want)}"
            got = to_host(send[r])
            assert np.array_equal(got, want), f"in place n={n} rank={r}: {first_mismatch(got, want)}"


@pytest.mark.parametrize("env,kw", POLICIES, ids=IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reduce_scatter_and_all_gather_each_policy(monkeypatch, env, kw, dtype):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    for R in (2, 5, 8):
        for L in (1, 5, 4099, 33333):
            n = L * R
            xs = rand(R, n, dtype, 91 * R + L)
            ref = oracle.reduce_scatter_ring(xs)
            send = [to_dev(x) for x in xs]
            recv = [torch.empty(L, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
            ws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc._dtype(send[0])), 16),
                             dtype=torch.uint8, device=send[0].device)
            hc.hc_reduce_scatter(send, recv, L, ws, **kw)
            torch.cuda.synchronize()
            for r in range(R):
                got = to_host(recv[r])
                assert np.array_equal(got, bits(ref[r])), f"RS R={R} L={L} rank={r}: {first_mismatch(got, bits(ref[r]))}"
            ys = [x[:L].copy() for x in xs]
            ref_ag = oracle.all_gather_ring(ys)
            outs = [torch.empty(L * R, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
            hc.hc_all_gather([to_dev(y) for y in ys], outs, L, **kw)
            torch.cuda.synchronize()
            for r in range(R):
                assert np.array_equal(to_host(outs[r]), bits(ref_ag[r])), f"AG R={R} L={L} rank={r}"


@pytest.mark.parametrize("env,kw", POLICIES, ids=IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_sgd_each_policy(monkeypatch, env, kw, dtype):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    for R in (1, 3, 8):
        for n in (7, 8192 * 3 + 17, 300_001):
            grads = rand(R, n, dtype, 13 * R + n, 1e-3)
            weights = rand(R, n, dtype, 17 * R + n, 1.0)
            ref = oracle.allreduce_sgd(grads, weights, 0.01)
            wd = [to_dev(w) for w in weights]
            hc.hc_allreduce_sgd([to_dev(g) for g in grads], wd, 0.01, **kw)
            torch.cuda.synchronize()
            for r in range(R):
                got = to_host(wd[r])
                assert np.array_equal(got, bits(ref[r])), f"R={R} n={n} rank={r}: {first_mismatch(got, bits(ref[r]))}"


def test_invalid_threshold_keeps_the_default(monkeypatch):
    """A value that is not a whole decimal number is ignored (the 320 MiB
    default applies); the call still succeeds with the oracle's values."""
    monkeypatch.setenv("HC_STREAM_STORE_MIN_BYTES", "12abc")
    R, n = 4, 65536 + 3
    xs = rand(R, n, "bf16", 8, 1e-3)
    ref = oracle.allreduce_fold(xs)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    hc.hc_allreduce(send, recv)
    torch.cuda.synchronize()
    for r in range(R):
        assert np.array_equal(to_host(recv[r]), bits(ref[r]))
