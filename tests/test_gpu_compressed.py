"""GPU parity of the fused compressed ring allreduce (hc_compressed_allreduce)
against the oracle: output bit-identical to the uncompressed ring (the codec
is lossless) and wire bytes equal to the oracle's count.

"CCCL: In-GPU Compression-Coupled Collective Communication", section 5
("Selective compression"), on the ring of "ResCCL: Resource-Efficient
Scheduling for Collective Communication" (section 1).

Allreduces up to HC_CHAIN_MAX_BYTES run as one launch in which each workgroup
carries one codec block of one slice through every hop; the tests run under
that default and with the threshold at 0 (one launch per ring step).  Both
schedules take the same hops in the same order, so the bits and the wire
bytes must not depend on the schedule."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu
B = 16384
SCHEDULES = [pytest.param({}, id="default"), pytest.param({"HC_CHAIN_MAX_BYTES": "0"}, id="steps"),
             pytest.param({"HC_CHAIN_MAX_BYTES": str(1 << 40)}, id="one_launch")]


def run_car(xs, inplace=False, chunk_fraction=0.0):
    R, n = len(xs), xs[0].size
    send = [to_dev(x) for x in xs]
    recv = send if inplace else [torch.empty_like(s) for s in send]
    ws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), 16), dtype=torch.uint8,
                     device="cuda")
    wire = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    hc.hc_compressed_allreduce(send, recv, n, ws, wire, chunk_fraction=chunk_fraction)
    torch.cuda.synchronize()
    return [to_host(t) for t in recv], int(wire.item())


@pytest.mark.parametrize("R,n", [(1, 1000), (2, 2 * B), (2, 7), (3, 3 * B + 300), (4, 8 * B), (5, 5 * B + 17),
                                 (8, 16 * B), (8, 64 * B + 8 * 1000 + 5), (7, 3)])
@pytest.mark.parametrize("schedule", SCHEDULES)
def test_compressed_allreduce_matches_oracle(monkeypatch, schedule, R, n):
    for k, v in schedule.items():
        monkeypatch.setenv(k, v)
    xs = [inputs.normal_bf16("test", 500 + r, n, 1e-3) for r in range(R)]
    ref = oracle.allreduce_fold(xs)
    chunk = oracle.chunk_elems(n, B)
    _, ref_wire = oracle.compressed_allreduce(xs, chunk=chunk)
    got, wire = run_car(xs)
    for r in range(R):
        assert np.array_equal(got[r], ref[r]), f"rank {r}: {first_mismatch(got[r], ref[r])}"
    assert wire == ref_wire


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_compressed_allreduce_in_place_and_chunking(monkeypatch, schedule):
    for k, v in schedule.items():
        monkeypatch.setenv(k, v)
    R, n = 4, 40 * B + 123
    xs = [inputs.normal_bf16("test", 600 + r, n, 1e-3) for r in range(R)]
    ref = oracle.allreduce_fold(xs)
    for frac in (0.0, 0.05, 1.0):
        chunk = oracle.chunk_elems(n, B) if frac == 0.0 else max(B, -(-int(np.ceil(n * frac)) // B) * B)
        _, ref_wire = oracle.compressed_allreduce(xs, chunk=chunk)
        for inplace in (False, True):
            got, wire = run_car(xs, inplace=inplace, chunk_fraction=frac)
            for r in range(R):
                assert np.array_equal(got[r], ref[r]), f"frac={frac} inplace={inplace} rank={r}"
            assert wire == ref_wire, f"frac={frac}"


@pytest.mark.timeout(600)
def test_compressed_allreduce_full_size_matches_oracle(monkeypatch):
    """R=8 x 2^25 bf16 N(0,1e-3): every element of every rank's output and
    the wire byte count equal the oracle's compressed ring (whose output is
    the uncompressed fold, bit for bit), and the compressed ring equals the
    uncompressed one on the GPU.  The one-launch schedule, forced at this
    size, gives the same bits and wire bytes."""
    R, n = 8, 1 << 25
    send = inputs.ring_inputs_cuda("compressed", R, n)
    xs = [inputs.host_bits(s) for s in send]
    out_c = [torch.empty_like(s) for s in send]
    out_u = [torch.empty_like(s) for s in send]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), dtype=torch.uint8, device="cuda")
    wire = torch.zeros(1, dtype=torch.int64, device="cuda")
    hc.hc_compressed_allreduce(send, out_c, n, ws, wire)
    hc.hc_allreduce(send, out_u)
    torch.cuda.synchronize()
    for r in range(R):
        assert torch.equal(out_c[r].view(torch.int16), out_u[r].view(torch.int16)), f"rank {r}"
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", str(1 << 40))
    wire1 = torch.zeros(1, dtype=torch.int64, device="cuda")
    hc.hc_compressed_allreduce(send, out_u, n, ws, wire1)
    torch.cuda.synchronize()
    for r in range(R):
        assert torch.equal(out_c[r].view(torch.int16), out_u[r].view(torch.int16)), f"one launch, rank {r}"
    assert int(wire1.item()) == int(wire.item())
    del send, out_u, ws
    torch.cuda.empty_cache()
    print("compressed ring equals the uncompressed ring; running the oracle", flush=True)
    ref, ref_wire = oracle.compressed_allreduce(xs, chunk=oracle.chunk_elems(n, B))
    for r in range(R):
        got = to_host(out_c[r])
        assert np.array_equal(got, ref[r]), f"rank {r}: {first_mismatch(got, ref[r])}"
    assert int(wire.item()) == ref_wire, (int(wire.item()), ref_wire)
    raw = 2 * (R - 1) * n * 2   # uncompressed wire bytes of the ring (both phases)
    assert 0.6 < ref_wire / raw < 0.8, ref_wire / raw


@pytest.mark.timeout(600)
@pytest.mark.parametrize("R,n", [(2, 1 << 28), (16, 1 << 22), (3, (1 << 26) + 12345)])
def test_one_launch_equals_step_schedule_at_scale(monkeypatch, R, n):
    """Beyond the oracle-checked sizes: the one-launch schedule gives the
    step schedule's bits and wire bytes at 2^28 elements per rank, at 16
    ranks, and with a ragged tail (the step schedule is itself checked
    against the oracle at R=8 x 2^25 above)."""
    send = inputs.ring_inputs_cuda("compressed", R, n)
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), dtype=torch.uint8, device="cuda")
    outs, wires = {}, {}
    for name, val in (("steps", "0"), ("one_launch", str(1 << 62))):
        monkeypatch.setenv("HC_CHAIN_MAX_BYTES", val)
        recv = [torch.empty_like(s) for s in send]
        wire = torch.zeros(1, dtype=torch.int64, device="cuda")
        hc.hc_compressed_allreduce(send, recv, n, ws, wire)
        torch.cuda.synchronize()
        outs[name], wires[name] = recv, int(wire.item())
    assert wires["steps"] == wires["one_launch"] > 0
    for r in range(R):
        assert torch.equal(outs["steps"][r].view(torch.int16), outs["one_launch"][r].view(torch.int16)), f"rank {r}"
    # every rank holds the same sums
    for r in range(1, R):
        assert torch.equal(outs["one_launch"][0].view(torch.int16), outs["one_launch"][r].view(torch.int16))
