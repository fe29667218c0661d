"""The ring collectives under HIP graph capture: an allreduce captured once
and replayed must give, on every replay, the result of the eager call on
the inputs of that moment.  The captured calls allocate nothing and issue no
memset; each replay is followed by eager work (new inputs copied in, a
synchronisation) before the next one, and every replay is checked."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from hc_util import bits, first_mismatch, to_host

pytestmark = pytest.mark.gpu


def rand(R, n, dtype, seed):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * (1e-3 if dtype == "bf16" else 1.0)).astype(np.float32) for _ in range(R)]
    if dtype == "bf16":
        from collective_communication_amd import inputs
        xs = [inputs.f32_to_bf16_bits(x) for x in xs]
    return xs


def load_into(dev_tensors, host_arrays):
    for t, x in zip(dev_tensors, host_arrays):
        src = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x.copy())
        t.copy_(src.view(t.dtype) if x.dtype == np.uint16 else src)


@pytest.mark.parametrize("op,dtype", [(op, dt) for op in ("allreduce", "allreduce_sgd", "reduce_scatter")
                                       for dt in ("f32", "bf16")] + [("allreduce_f32carry", "bf16")])
def test_captured_collective_replays_match_eager(op, dtype):
    R, n = 8, 8 * 12345 + 3 if op != "reduce_scatter" else 8 * 12345
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    send = [torch.empty(n, dtype=tdt, device="cuda") for _ in range(R)]
    weights = [torch.empty(n, dtype=tdt, device="cuda") for _ in range(R)]
    L = n // R
    recv = ([torch.empty(L, dtype=tdt, device="cuda") for _ in range(R)] if op == "reduce_scatter"
            else [torch.empty(n, dtype=tdt, device="cuda") for _ in range(R)])
    ws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc._dtype(send[0])), 16),
                     dtype=torch.uint8, device="cuda")

    cws = None
    if op == "allreduce_f32carry":
        cws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, n, R, hc.HC_BF16), dtype=torch.uint8,
                          device="cuda")

    def call():
        if op == "allreduce":
            hc.hc_allreduce(send, recv)
        elif op == "allreduce_f32carry":
            hc.hc_allreduce_bf16_f32carry(send, recv, n, cws)
        elif op == "allreduce_sgd":
            hc.hc_allreduce_sgd(send, weights, 0.01)
        else:
            hc.hc_reduce_scatter(send, recv, L, ws)

    load_into(send, rand(R, n, dtype, 1))
    load_into(weights, rand(R, n, dtype, 2))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()   # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for k in range(4):
        xs = rand(R, n, dtype, 10 + k)
        ws_host = rand(R, n, dtype, 20 + k)
        load_into(send, xs)
        load_into(weights, ws_host)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if op == "allreduce":
            ref = oracle.allreduce_fold(xs)
            outs = recv
        elif op == "allreduce_f32carry":
            ref = oracle.allreduce_fold_f32carry(xs)
            outs = recv
        elif op == "allreduce_sgd":
            ref = oracle.allreduce_sgd(xs, ws_host, 0.01)
            outs = weights
        else:
            ref = oracle.reduce_scatter_ring(xs)
            outs = recv
        for r in range(R):
            got = to_host(outs[r])
            assert np.array_equal(got, bits(ref[r])), f"replay {k} rank {r}: {first_mismatch(got, bits(ref[r]))}"


@pytest.mark.parametrize("chain_max", ["0", str(1 << 40)], ids=["steps", "one_launch"])
def test_captured_compressed_allreduce_and_codec_replays(monkeypatch, chain_max):
    """The compressed allreduce and the stream codec (ticket counters and
    look-back descriptors cleared by a fill kernel inside the launch) replayed
    from one graph: the wire bytes, the sums, the stream and its decode match
    the oracle on every replay."""
    from collective_communication_amd import inputs
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", chain_max)
    B = 16384
    R, n = 4, 3 * B + 517
    send = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    recv = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    ws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), 16), dtype=torch.uint8,
                     device="cuda")
    wire = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cap = hc.hc_compress_bound_bf16(n)
    stream = torch.empty(cap, dtype=torch.uint8, device="cuda")
    cws = torch.empty(max(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), 16), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")

    def call():
        hc.hc_compressed_allreduce(send, recv, n, ws, wire)
        hc.hc_compress_bf16(send[0], n, stream, size, cws)
        hc.hc_decompress_bf16(stream, cap, back, n, status)

    load_into(send, [inputs.normal_bf16("test", 300 + r, n, 1e-3) for r in range(R)])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for k in range(4):
        xs = [inputs.normal_bf16("test", 400 + 10 * k + r, n, 10.0 ** -(1 + k)) for r in range(R)]
        load_into(send, xs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.allreduce_fold(xs)
        _, ref_wire = oracle.compressed_allreduce(xs, chunk=oracle.chunk_elems(n, B))
        for r in range(R):
            assert np.array_equal(to_host(recv[r]), ref[r]), f"replay {k} rank {r}"
        assert int(wire.item()) == ref_wire, f"replay {k}: wire bytes"
        ref_stream = oracle.compress(xs[0])
        m = int(size.item())
        assert m == len(ref_stream), f"replay {k}: stream size {m} vs {len(ref_stream)}"
        assert to_host(stream)[:m].tobytes() == ref_stream, f"replay {k}: stream bytes"
        assert int(status.item()) == 0 and np.array_equal(to_host(back), xs[0]), f"replay {k}: decode"
