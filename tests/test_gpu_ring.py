"""GPU parity of the ring reduce-scatter / all-gather / allreduce (libhc,
gfx950) against the oracle, bit for bit.

Ring: "ResCCL: Resource-Efficient Scheduling for Collective Communication"
(section 1, recvReduceCopy and copy hops, ~1% chunks); AllReduce =
ReduceScatter then AllGather ("Breaking the computation and communication
abstraction barrier in distributed machine learning workloads", "The idea").
The fold order is fixed, so the bar is bit-exact for fp32 and bf16."""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import bits, copy_engine_or_unsupported, first_mismatch, fold_chunked, to_dev, to_host

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def rand(R, n, dtype, seed, scale=1.0):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * scale).astype(np.float32) for _ in range(R)]
    if dtype == "bf16":
        xs = [inputs.f32_to_bf16_bits(x) for x in xs]
    return xs


def run_ar(xs, inplace=False, **kw):
    send = [to_dev(x) for x in xs]
    recv = send if inplace else [torch.empty_like(s) for s in send]
    hc.hc_allreduce(send, recv, **kw)
    torch.cuda.synchronize()
    return [to_host(t) for t in recv]


SIZES = [1, 7, 8, 64, 1000, 8192 * 3 + 17, 65536, 300_001]


# Allreduces up to HC_CHAIN_MAX_BYTES (256 MiB by default) run as one launch that
# carries each tile through every hop; larger ones launch once per ring step.
# Both schedules are run on the small shapes.
SCHEDULES = [pytest.param({}, id="default"), pytest.param({"HC_CHAIN_MAX_BYTES": "0"}, id="steps")]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8])
def test_allreduce_matches_oracle(monkeypatch, schedule, dtype, R):
    for k, v in schedule.items():
        monkeypatch.setenv(k, v)
    for n in SIZES:
        xs = rand(R, n, dtype, 1000 * R + n, 1e-3 if dtype == "bf16" else 1.0)
        ref = oracle.allreduce_fold(xs)
        got = run_ar(xs)
        for r in range(R):
            assert np.array_equal(got[r], bits(ref[r])), f"n={n} rank={r}: {first_mismatch(got[r], bits(ref[r]))}"


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_allreduce_in_place_and_chunk_independent(monkeypatch, schedule, dtype):
    for k, v in schedule.items():
        monkeypatch.setenv(k, v)
    R, n = 8, 8 * 40000 + 24
    xs = rand(R, n, dtype, 5)
    ref = oracle.allreduce_fold(xs)
    for kw in ({"inplace": True}, {"chunk_fraction": 0.001}, {"chunk_fraction": 0.37},
               {"chunk_fraction": 1.0}, {"cu_budget": 8}, {"cu_budget": 32},
               {"copy_engine": 1}, {"copy_engine": 1, "inplace": True, "chunk_fraction": 0.01}):
        if kw.get("copy_engine"):
            out = []
            if not copy_engine_or_unsupported(lambda: out.append(run_ar(xs, **kw))):
                continue
            got = out[0]
        else:
            got = run_ar(xs, **kw)
        for r in range(R):
            assert np.array_equal(got[r], bits(ref[r])), f"{kw} rank={r}: {first_mismatch(got[r], bits(ref[r]))}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_reduce_scatter_matches_oracle(dtype, R):
    for L in (1, 5, 1024, 33333):
        n = L * R
        xs = rand(R, n, dtype, 77 * R + L)
        ref = oracle.reduce_scatter_ring(xs)
        send = [to_dev(x) for x in xs]
        recv = [torch.empty(L, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
        ws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc._dtype(send[0])), 16),
                         dtype=torch.uint8, device=send[0].device)
        hc.hc_reduce_scatter(send, recv, L, ws)
        torch.cuda.synchronize()
        for r in range(R):
            got = to_host(recv[r])
            assert np.array_equal(got, bits(ref[r])), f"L={L} rank={r}: {first_mismatch(got, bits(ref[r]))}"
        # in place: rank r's output is slice r of its own input
        hc.hc_reduce_scatter(send, [s[r * L:(r + 1) * L] for r, s in enumerate(send)], L, ws)
        torch.cuda.synchronize()
        for r in range(R):
            got = to_host(send[r][r * L:(r + 1) * L])
            assert np.array_equal(got, bits(ref[r])), f"in-place L={L} rank={r}"


@pytest.mark.parametrize("copy_engine", [0, 1], ids=["cu", "dma"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 5, 8])
def test_all_gather_matches_oracle(dtype, R, copy_engine):
    """copy_engine=1: the copies run on the DMA engines (no compute unit), or
    the call refuses where the runtime would not offload them."""
    for L in (1, 3, 4096, 20001):
        xs = rand(R, L, dtype, 3 * R + L)
        ref = oracle.all_gather_ring(xs)
        send = [to_dev(x) for x in xs]
        recv = [torch.empty(L * R, dtype=send[0].dtype, device=send[0].device) for _ in range(R)]
        if copy_engine and not copy_engine_or_unsupported(lambda: hc.hc_all_gather(send, recv, L, copy_engine=1)):
            return
        if not copy_engine:
            hc.hc_all_gather(send, recv, L, copy_engine=copy_engine)
        torch.cuda.synchronize()
        for r in range(R):
            assert np.array_equal(to_host(recv[r]), bits(ref[r])), f"L={L} rank={r}"
        # in place: the send buffer is slice r of the output
        outs = [to_dev(np.zeros(L * R, dtype=xs[0].dtype)) for _ in range(R)]
        for r in range(R):
            outs[r][r * L:(r + 1) * L].copy_(send[r])
        hc.hc_all_gather([o[r * L:(r + 1) * L] for r, o in enumerate(outs)], outs, L, copy_engine=copy_engine)
        torch.cuda.synchronize()
        for r in range(R):
            assert np.array_equal(to_host(outs[r]), bits(ref[r])), f"in-place L={L} rank={r}"


def test_bf16_hop_every_a_against_sampled_b():
    """R=2 allreduce: slice 0 computes hop(x1, x0), slice 1 hop(x0, x1), one fp32
    add and one bf16 rounding each, over all 65,536 bf16 patterns of one operand."""
    g = np.random.default_rng(21)
    a = np.arange(1 << 16, dtype=np.uint16)
    for bv in list(g.integers(0, 1 << 16, 24)) + [0x0000, 0x8000, 0x0001, 0x7F7F, 0x7F80, 0xFF80, 0x7FC0, 0xFFFF]:
        b = np.full(a.size, bv, dtype=np.uint16)
        got = run_ar([a, b])
        want = oracle.hop_bf16_array(b, a)[: a.size // 2]
        want = np.concatenate([want, oracle.hop_bf16_array(a, b)[a.size // 2:]])
        assert np.array_equal(got[0], want), f"b=0x{int(bv):04x}: {first_mismatch(got[0], want)}"


def test_fp32_hop_specials_and_subnormals():
    g = np.random.default_rng(22)
    a = g.integers(0, 1 << 32, 1 << 16, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000,
                        0xFF800000, 0x7FC00000, 0xFFC00001, 0x3F800000], dtype=np.uint32)
    a[:special.size] = special
    b = np.roll(a, 7)
    got = run_ar([a.view(np.float32), b.view(np.float32)])
    half = a.size // 2
    want = np.concatenate([oracle.hop_f32_array(b, a)[:half], oracle.hop_f32_array(a, b)[half:]])
    assert np.array_equal(got[0], want), first_mismatch(got[0], want)


def test_ring_f32_workload_full_size():
    """R=4 x 2^20 fp32 N(0,1), every rank's output equals the oracle's."""
    xs = [inputs.host_bits(t) for t in inputs.ring_inputs_cuda("ring_f32", 4, 1 << 20)]
    ref = oracle.allreduce_fold(xs)
    got = run_ar(xs)
    for r in range(4):
        assert np.array_equal(got[r], bits(ref[r])), first_mismatch(got[r], bits(ref[r]))


def test_ring_bf16_workload_full_size():
    """R=8 x 2^26 bf16 N(0,1e-3) with 1% zeros: every element of every rank's
    output equals the oracle's fold."""
    R, n = 8, 1 << 26
    send = inputs.ring_inputs_cuda("ring_bf16", R, n)
    xs = [inputs.host_bits(s) for s in send]
    recv = [torch.empty_like(s) for s in send]
    hc.hc_allreduce(send, recv)
    torch.cuda.synchronize()
    del send
    want = fold_chunked(xs)
    for r in range(R):
        got = to_host(recv[r])
        assert np.array_equal(got, want), f"rank {r}: {first_mismatch(got, want)}"
    del recv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 3, 8])
def test_allreduce_copy_engine_matches_oracle(dtype, R):
    """Reduce-scatter on the compute units, all-gather on the DMA engines (or a
    refusal where this process's runtime would not offload the copies)."""
    for n in (1, 1000, 65536 + 5):
        xs = rand(R, n, dtype, 4242 * R + n, 1e-3 if dtype == "bf16" else 1.0)
        ref = oracle.allreduce_fold(xs)
        out = []
        if not copy_engine_or_unsupported(lambda: out.append(run_ar(xs, copy_engine=1))):
            return
        got = out[0]
        for r in range(R):
            assert np.array_equal(got[r], bits(ref[r])), f"n={n} rank={r}: {first_mismatch(got[r], bits(ref[r]))}"


def test_all_gather_copy_engine_under_system_runtime(tmp_path):
    """copy_engine=1 in a process on the system ROCm runtime (dma_contention,
    no torch): the all-gather of seeded inputs written here equals the
    oracle's all-gather byte for byte, and it completes while a bounded kernel
    holds every wave slot of the GPU, i.e. it used no compute unit.  A second
    run checks the tool's own copy-kernel comparison.  (Inside a torch process
    the HIP runtime bundled with the wheel would serve the same calls with
    blit kernels, so there the library refuses copy_engine=1.)"""
    tool = os.path.join(ROOT, "measure", "dma_contention")
    assert os.path.exists(tool), "dma_contention is not built"
    R, L = 8, 65536 + 3
    xs = [inputs.normal_bf16("test", 8800 + r, L, 1e-3) for r in range(R)]
    want = oracle.all_gather_ring(xs)
    (tmp_path / "meta.txt").write_text(f"{R} {L}\n")
    for r in range(R):
        xs[r].astype("<u2").tofile(tmp_path / f"in_{r}.bin")
        want[r].astype("<u2").tofile(tmp_path / f"expected_{r}.bin")
    r = subprocess.run([tool, "verify", str(tmp_path)], capture_output=True, text=True, timeout=120)
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["against"] == "expected files" and line["mismatched_words"] == 0, line
    assert line["no_compute_units"] is True, line
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([tool, "verify"], capture_output=True, text=True, timeout=120)
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["mismatched_words"] == 0 and line["no_compute_units"] is True and r.returncode == 0, line


def test_copy_engine_refused_where_it_would_use_compute_units():
    """In this (torch) process: copy_engine=1 either runs on the DMA engines
    (a runtime of 7.2 or later) or is refused before anything is enqueued."""
    import ctypes

    L = hc.load()
    v = ctypes.c_int(0)
    assert ctypes.CDLL("libamdhip64.so.7").hipRuntimeGetVersion(ctypes.byref(v)) == 0
    assert hc.hc_copy_engine_available() == (v.value >= 70200000), v.value
    xs = rand(3, 999, "bf16", 17)
    send = [to_dev(x) for x in xs]
    recv = [torch.full_like(s, 7.0) for s in send]
    ran = copy_engine_or_unsupported(lambda: hc.hc_allreduce(send, recv, copy_engine=1))
    torch.cuda.synchronize()
    if not ran:   # nothing was enqueued
        assert all(bool((t == 7.0).all()) for t in recv)
    assert L.hc_copy_engine_available() in (0, 1)


def test_hbm_ceiling_tool():
    """The streaming-ceiling tool (the bar the reduce hop is held against next
    to the published peak) runs and reports every mix with its bytes."""
    tool = os.path.join(ROOT, "measure", "hbm_ceiling")
    assert os.path.exists(tool), "hbm_ceiling is not built"
    r = subprocess.run([tool, "64", "3"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["operand_bytes"] == 64 << 20
    for mix, ops in (("add", 3), ("copy", 2), ("read", 2)):
        assert line[mix]["bytes"] == ops * (64 << 20) and line[mix]["gbps"] > 0 and line[mix]["us"] > 0, line
    assert subprocess.run([tool, "0"], capture_output=True, timeout=60).returncode == 2


@pytest.mark.timeout(900)
def test_reduce_scatter_contention_workload_full_size():
    """The contention workload's reduce-scatter, R=8 x 2^28 bf16 N(0,1e-3) with
    1% zeros, on all CUs and on a stream masked to 8 CUs (the persistent
    grid): both launches give the same bytes, and every element of every
    rank's slice equals the oracle's fold."""
    R, n = 8, 1 << 28
    L = n // R
    send = inputs.ring_inputs_cuda("contention", R, n)
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    recv = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    hc.hc_reduce_scatter(send, recv, L, ws)
    torch.cuda.synchronize()
    handle = hc.hc_stream_create_cu_budget(8)
    try:
        side = torch.cuda.ExternalStream(handle)
        masked = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        hc.hc_reduce_scatter(send, masked, L, ws, cu_budget=8, stream=side)
        side.synchronize()
        del side
    finally:
        hc.hc_stream_destroy(handle)
    for r in range(R):
        assert torch.equal(masked[r].view(torch.int16), recv[r].view(torch.int16)), f"rank {r}: cu_budget 8 differs"
    xs = [inputs.host_bits(t) for t in send]
    del send, masked, ws
    torch.cuda.empty_cache()
    for r in range(R):
        want = fold_chunked(xs, r * L, (r + 1) * L)
        got = to_host(recv[r])
        assert np.array_equal(got, want), f"rank {r}: {first_mismatch(got, want)}"
        print(f"contention reduce-scatter: rank {r} slice equals the oracle", flush=True)
    del recv
    torch.cuda.empty_cache()
