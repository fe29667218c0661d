"""Kernel-stamped step events (hc_opts_t.step_event_mode 1): every ring step's
kernels stamp two events with their own start and end.  The stamps must come
in stream order, fit inside the call, leave every value unchanged (bit-exact
against the oracle), cover steps without a kernel (the all-gather step that
the last reduce-scatter step already did, copy-engine copies), and leave no
stamp open for a later call."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import copy_engine_or_unsupported, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu

N = 8 * 4096 * 40 + 11   # several tiles per receiver and a ragged tail


def rand_bf16(R, n, seed, scale=1e-3):
    g = np.random.default_rng(seed)
    return [inputs.f32_to_bf16_bits((g.standard_normal(n) * scale).astype(np.float32)) for _ in range(R)]


def stamped(call, steps):
    """Runs call(step_events) between two outer events; checks the stamps and
    returns the per-step durations (ms)."""
    ev = hc.StepEvents.for_steps(steps, mode=1)
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    outer[0].record()
    call(ev)
    outer[1].record()
    torch.cuda.synchronize()
    d = ev.elapsed_ms()
    assert len(d) == steps
    assert all(t >= 0 for t in d), d
    e = ev.events
    for k in range(steps - 1):   # step k ends before step k+1 starts
        assert e[2 * k + 1].elapsed_time(e[2 * k + 2]) >= -1e-3, k
    assert outer[0].elapsed_time(e[0]) >= -1e-3
    assert e[-1].elapsed_time(outer[1]) >= -1e-3
    assert sum(d) <= outer[0].elapsed_time(outer[1]) + 1e-3
    return d, ev


def check(got, ref, label):
    for r in range(len(ref)):
        assert np.array_equal(got[r], ref[r]), f"{label} rank {r}: {first_mismatch(got[r], ref[r])}"


@pytest.mark.parametrize("copy_engine", [0, 1])
def test_allreduce(copy_engine):
    R = 8
    xs = rand_bf16(R, N, 11 + copy_engine)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE, R)
    if copy_engine and not copy_engine_or_unsupported(
            lambda: stamped(lambda ev: hc.hc_allreduce(send, recv, step_events=ev, copy_engine=1), steps)):
        return   # this process's runtime would not offload the copies: the call refused
    d, _ = stamped(lambda ev: hc.hc_allreduce(send, recv, step_events=ev, copy_engine=copy_engine), steps)
    check([to_host(t) for t in recv], oracle.allreduce_fold(xs), f"copy_engine {copy_engine}")
    assert all(t > 0 for t in d[:R - 1])          # reduce-scatter kernels
    if copy_engine:
        assert all(t > 0 for t in d[R - 1:])      # every all-gather step copies on the engines


def test_no_stamp_left_open():
    # A plain call after a stamped one must not re-stamp the stamped call's events.
    R = 4
    xs = rand_bf16(R, N, 21)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE, R)
    d, ev = stamped(lambda ev: hc.hc_allreduce(send, recv, step_events=ev), steps)
    for _ in range(3):
        hc.hc_allreduce(send, recv)
        hc.hc_allreduce_bf16_f32carry(send, recv, N, torch.empty(
            hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, N, R, hc.HC_BF16), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert ev.elapsed_ms() == d


def test_carry_and_sgd():
    R = 8
    xs = rand_bf16(R, N, 31)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, N, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE_F32_CARRY, R)
    stamped(lambda ev: hc.hc_allreduce_bf16_f32carry(send, recv, N, ws, step_events=ev), steps)
    check([to_host(t) for t in recv], oracle.allreduce_fold_f32carry(xs), "f32 carry")

    w0 = rand_bf16(1, N, 32, 1.0)[0]
    weights = [to_dev(w0) for _ in range(R)]
    grads = [to_dev(x) for x in xs]
    stamped(lambda ev: hc.hc_allreduce_sgd(grads, weights, 0.25, step_events=ev),
            hc.hc_step_count(hc.HC_OP_ALLREDUCE, R))
    check([to_host(w) for w in weights], oracle.allreduce_sgd(xs, [w0] * R, 0.25), "sgd")


def test_reduce_scatter_all_gather_and_one_rank():
    R, L = 4, 100003
    xs = rand_bf16(R, R * L, 41)
    send = [to_dev(x) for x in xs]
    out = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, R * L, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    stamped(lambda ev: hc.hc_reduce_scatter(send, out, L, ws, step_events=ev),
            hc.hc_step_count(hc.HC_OP_REDUCE_SCATTER, R))
    check([to_host(t) for t in out], oracle.reduce_scatter_ring(xs), "reduce-scatter")

    parts = [to_dev(x[:L]) for x in xs]
    full = [torch.empty(R * L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    stamped(lambda ev: hc.hc_all_gather(parts, full, L, step_events=ev), hc.hc_step_count(hc.HC_OP_ALL_GATHER, R))
    check([to_host(t) for t in full], oracle.all_gather_ring([x[:L] for x in xs]), "all-gather")

    one = [to_dev(xs[0])]
    dst = [torch.empty_like(one[0])]
    d, _ = stamped(lambda ev: hc.hc_allreduce(one, dst, step_events=ev), 1)
    assert d[0] > 0 and np.array_equal(to_host(dst[0]), xs[0])


def test_compressed_allreduce():
    R, n = 4, 3 * 16384 * 4 + 777
    xs = rand_bf16(R, n, 51)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), dtype=torch.uint8, device="cuda")
    d, _ = stamped(lambda ev: hc.hc_compressed_allreduce(send, recv, n, ws, step_events=ev),
                   hc.hc_step_count(hc.HC_OP_COMPRESSED_ALLREDUCE, R))
    assert all(t > 0 for t in d)
    ref, _ = oracle.compressed_allreduce(xs)
    check([to_host(t) for t in recv], ref, "compressed")
