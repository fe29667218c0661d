"""GPU parity of the allreduce fused with an SGD update (libhc,
hc_allreduce_sgd) against the oracle, bit for bit.

"Breaking the computation and communication abstraction barrier in
distributed machine learning workloads" ("The idea"): the optimizer update
sits between the ReduceScatter and the AllGather, on each rank's slice.  The
sum is the ring fold of hc_allreduce and the update rounds the product and
the difference once each, so the bar is bit-exact for fp32 and bf16."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import copy_engine_or_unsupported, bits, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def rand(R, n, dtype, seed, scale):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * scale).astype(np.float32) for _ in range(R)]
    if dtype == "bf16":
        xs = [inputs.f32_to_bf16_bits(x) for x in xs]
    return xs


def run(grads, weights, lr, **kw):
    gd = [to_dev(x) for x in grads]
    wd = [to_dev(x) for x in weights]
    hc.hc_allreduce_sgd(gd, wd, lr, **kw)
    torch.cuda.synchronize()
    return [to_host(t) for t in wd]


SIZES = [1, 7, 64, 1000, 8192 * 3 + 17, 65536, 300_001]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 5, 8])
def test_allreduce_sgd_matches_oracle(dtype, R):
    for n in SIZES:
        grads = rand(R, n, dtype, 31 * R + n, 1e-3)
        weights = rand(R, n, dtype, 37 * R + n, 1.0)    # every rank different: the owner's slice counts
        ref = oracle.allreduce_sgd(grads, weights, 0.01)
        got = run(grads, weights, 0.01)
        for r in range(R):
            assert np.array_equal(got[r], bits(ref[r])), f"n={n} rank={r}: {first_mismatch(got[r], bits(ref[r]))}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_sgd_options_change_no_value(dtype):
    R, n = 8, 8 * 40000 + 24
    grads = rand(R, n, dtype, 5, 1e-2)
    w0 = rand(1, n, dtype, 6, 1.0)[0]
    weights = [w0.copy() for _ in range(R)]                 # data-parallel: replicated weights
    ref = oracle.allreduce_sgd(grads, weights, 0.5)
    for kw in ({}, {"chunk_fraction": 0.001}, {"chunk_fraction": 1.0}, {"cu_budget": 8},
               {"copy_engine": 1}):
        if kw.get("copy_engine"):
            out = []
            if not copy_engine_or_unsupported(lambda: out.append(run(grads, weights, 0.5, **kw))):
                continue
            got = out[0]
        else:
            got = run(grads, weights, 0.5, **kw)
        for r in range(R):
            assert np.array_equal(got[r], bits(ref[r])), f"{kw} rank={r}: {first_mismatch(got[r], bits(ref[r]))}"


def test_allreduce_sgd_step_events():
    R, n = 4, 1 << 16
    grads = rand(R, n, "bf16", 8, 1e-3)
    weights = rand(R, n, "bf16", 9, 1.0)
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE, R)
    ev = hc.StepEvents([torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)])
    got = run(grads, weights, 0.1, step_events=ev)
    ref = oracle.allreduce_sgd(grads, weights, 0.1)
    assert np.array_equal(got[0], ref[0])
    assert len(ev.elapsed_ms()) == steps and all(t >= 0 for t in ev.elapsed_ms())


def test_allreduce_sgd_full_size_sampled():
    """R=8 x 2^26 bf16 (the ring workload's shape), checked at 8192 sampled
    elements per rank plus every slice boundary against the oracle's fold and
    update rule."""
    R, n, lr = 8, 1 << 26, 0.01
    grads = inputs.ring_inputs_cuda("ring_bf16", R, n)
    w = inputs.normal_bf16_cuda("fused_sgd", 0, n, 1.0)
    weights = [w.clone() for _ in range(R)]
    g = np.random.default_rng(3)
    L = n // R
    idx = np.unique(np.concatenate([g.integers(0, n, 8192), np.arange(R) * L, np.arange(1, R + 1) * L - 1]))
    it = torch.from_numpy(idx.astype(np.int64)).cuda()
    gs = [inputs.host_bits(t.index_select(0, it)) for t in grads]
    w_at = inputs.host_bits(w.index_select(0, it))
    hc.hc_allreduce_sgd(grads, weights, lr)
    torch.cuda.synchronize()
    # the fold at each sampled index (ranks j+1, ..., j in ring order), then the update
    full_sum = []
    for k, i in enumerate(idx):
        j = int(i) // L
        acc = int(gs[(j + 1) % R][k])
        for t in range(2, R + 1):
            acc = oracle.hop_bf16(acc, int(gs[(j + t) % R][k]))
        full_sum.append(oracle.sgd_bf16(int(w_at[k]), acc, lr))
    want = np.array(full_sum, dtype=np.uint16)
    for r in range(R):
        got = inputs.host_bits(weights[r].index_select(0, it))
        assert np.array_equal(got, want), f"rank {r}: {first_mismatch(got, want)}"
