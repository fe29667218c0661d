"""Guard bands around every buffer a call writes: the bytes just before and
just after each output, workspace, byte counter and compressed stream hold a
known pattern, and after the call (checked against the oracle) none of them
has changed.  For the codecs the band after a stream starts at its size: the
bytes in [size, capacity) of the output must be left as they were.  This is
the race and overrun check of the test plan: a kernel that writes one
element, one vector or one record past what it owns fails here even when its
own output is right."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import bits, first_mismatch, to_host

pytestmark = pytest.mark.gpu
B = 16384
FILL = 0xA5


class Guarded:
    """A device buffer of nbytes bytes with `guard` bytes of FILL on both
    sides; the middle starts 256-byte aligned and may be prefilled too."""

    def __init__(self, nbytes: int, guard: int = 1 << 16, fill_middle: bool = True):
        self.nbytes, self.guard = nbytes, guard
        self.buf = torch.full((2 * guard + nbytes,), FILL, dtype=torch.uint8, device="cuda")
        if not fill_middle:
            self.buf[guard:guard + nbytes].zero_()

    def bytes(self) -> torch.Tensor:
        return self.buf[self.guard:self.guard + self.nbytes]

    def view(self, dtype) -> torch.Tensor:
        return self.bytes().view(dtype)

    def check(self, name: str, valid: int | None = None):
        """The bands outside [0, valid) (valid defaults to the whole middle)
        still hold FILL."""
        v = self.nbytes if valid is None else valid
        h = self.buf.cpu().numpy()
        before = h[:self.guard]
        after = h[self.guard + v:]
        bad_b = np.nonzero(before != FILL)[0]
        bad_a = np.nonzero(after != FILL)[0]
        assert bad_b.size == 0, f"{name}: {bad_b.size} bytes before the buffer changed, last at -{self.guard - bad_b[-1]}"
        assert bad_a.size == 0, f"{name}: {bad_a.size} bytes from offset {v} changed, first at +{bad_a[0]}"


def guarded_from(x: np.ndarray) -> Guarded:
    g = Guarded(x.nbytes)
    g.bytes().copy_(torch.from_numpy(x.view(np.uint8).copy()))
    return g


def tdtype(x: np.ndarray):
    return torch.bfloat16 if x.dtype == np.uint16 else torch.float32


def rand(R, n, dtype, seed):
    if dtype == "bf16":
        return [inputs.normal_bf16("test", seed + r, n, 1e-3) for r in range(R)]
    return [inputs.normal_f32("test", seed + r, n) for r in range(R)]


@pytest.mark.parametrize("dtype,R,n", [("bf16", 3, 3 * 1000 + 7), ("f32", 5, 4099), ("bf16", 8, 8 * 4096 + 5),
                                       ("bf16", 2, 1), ("f32", 64, 65 * 64 + 3)])
@pytest.mark.parametrize("inplace", [False, True])
def test_allreduce_writes_nothing_outside_its_outputs(dtype, R, n, inplace):
    xs = rand(R, n, dtype, 9100 + R)
    send = [guarded_from(x) for x in xs]
    recv = send if inplace else [Guarded(xs[0].nbytes) for _ in range(R)]
    td = tdtype(xs[0])
    hc.hc_allreduce([s.view(td) for s in send], [r.view(td) for r in recv])
    torch.cuda.synchronize()
    ref = oracle.allreduce_fold(xs)
    for r in range(R):
        got = to_host(recv[r].view(td))
        assert np.array_equal(got, bits(ref[r])), f"rank {r}: {first_mismatch(got, bits(ref[r]))}"
        recv[r].check(f"recvbufs[{r}]")
        send[r].check(f"sendbufs[{r}]")


@pytest.mark.parametrize("dtype,R,L", [("bf16", 4, 3001), ("f32", 3, 777), ("bf16", 8, 8192)])
def test_reduce_scatter_and_all_gather_write_nothing_outside(dtype, R, L):
    n = R * L
    xs = rand(R, n, dtype, 9200 + R)
    td = tdtype(xs[0])
    es = xs[0].itemsize
    send = [guarded_from(x) for x in xs]
    recv = [Guarded(L * es) for _ in range(R)]
    ws = Guarded(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc.HC_F32 if dtype == "f32" else hc.HC_BF16))
    hc.hc_reduce_scatter([s.view(td) for s in send], [r.view(td) for r in recv], L, ws.bytes())
    torch.cuda.synchronize()
    ref = oracle.allreduce_fold(xs)[0]
    for r in range(R):
        got = to_host(recv[r].view(td))
        want = bits(ref[r * L:(r + 1) * L])
        assert np.array_equal(got, want), f"rank {r}: {first_mismatch(got, want)}"
        recv[r].check(f"reduce-scatter recvbufs[{r}]")
    ws.check("reduce-scatter workspace")
    # all-gather of the slices
    gat = [Guarded(n * es) for _ in range(R)]
    hc.hc_all_gather([r.view(td) for r in recv], [g.view(td) for g in gat], L)
    torch.cuda.synchronize()
    for r in range(R):
        got = to_host(gat[r].view(td))
        assert np.array_equal(got, bits(ref)), f"all-gather rank {r}: {first_mismatch(got, bits(ref))}"
        gat[r].check(f"all-gather recvbufs[{r}]")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_allreduce_sgd_writes_nothing_outside(dtype):
    R, n = 4, 5003
    gs = rand(R, n, dtype, 9300)
    w0 = rand(1, n, dtype, 9400)[0]
    td = tdtype(gs[0])
    grads = [guarded_from(x) for x in gs]
    weights = [guarded_from(w0) for _ in range(R)]
    hc.hc_allreduce_sgd([g.view(td) for g in grads], [w.view(td) for w in weights], 0.01)
    torch.cuda.synchronize()
    ref = oracle.allreduce_sgd(gs, [w0] * R, 0.01)
    for r in range(R):
        got = to_host(weights[r].view(td))
        assert np.array_equal(got, bits(ref[r])), f"rank {r}: {first_mismatch(got, bits(ref[r]))}"
        weights[r].check(f"weights[{r}]")
        grads[r].check(f"grads[{r}]")


def test_f32carry_writes_nothing_outside():
    R, n = 5, 9999
    xs = rand(R, n, "bf16", 9500)
    send = [guarded_from(x) for x in xs]
    recv = [Guarded(2 * n) for _ in range(R)]
    ws = Guarded(hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, n, R, hc.HC_BF16))
    hc.hc_allreduce_bf16_f32carry([s.view(torch.bfloat16) for s in send], [r.view(torch.bfloat16) for r in recv],
                                  n, ws.bytes())
    torch.cuda.synchronize()
    ref = oracle.allreduce_fold_f32carry(xs)
    for r in range(R):
        got = to_host(recv[r].view(torch.bfloat16))
        assert np.array_equal(got, ref[r]), f"rank {r}: {first_mismatch(got, ref[r])}"
        recv[r].check(f"recvbufs[{r}]")
    ws.check("fp32-carry workspace")


CODERS = {
    "hcz1": (hc.hc_compress_bf16, hc.hc_decompress_bf16, hc.HC_OP_COMPRESS, oracle.compress),
    "staged": (hc.hc_compress_bf16_staged, hc.hc_decompress_bf16, hc.HC_OP_COMPRESS_STAGED, oracle.compress),
    "hce1": (hc.hc_compress_bf16_entropy, hc.hc_decompress_bf16_entropy, hc.HC_OP_COMPRESS_ENTROPY,
             oracle.hce_compress),
}


@pytest.mark.parametrize("coder", sorted(CODERS))
@pytest.mark.parametrize("n", [0, 5, B, 3 * B + 5, 20 * B])
def test_codec_writes_nothing_past_the_stream(coder, n):
    comp, decomp, op, ref_comp = CODERS[coder]
    x = inputs.normal_bf16("test", 9600 + n, n, 0.02) if n else np.zeros(0, dtype=np.uint16)
    cap = hc.hc_compress_bound_bf16(n)
    src = guarded_from(x) if n else Guarded(16)
    out = Guarded(cap)
    nbytes = Guarded(8)
    ws = Guarded(max(hc.hc_workspace_bytes(op, n, 1), 16))
    comp(src.view(torch.int16) if n else torch.zeros(8, dtype=torch.int16, device="cuda"), n, out.bytes(),
         nbytes.view(torch.int64), ws.bytes())
    torch.cuda.synchronize()
    size = int(nbytes.view(torch.int64).item())
    want = ref_comp(x)
    assert size == len(want)
    assert out.bytes()[:size].cpu().numpy().tobytes() == want
    out.check("stream output", valid=size)
    nbytes.check("byte count")
    ws.check("workspace")
    if n:
        src.check("input")
    back = Guarded(2 * n if n else 16)
    status = Guarded(4)
    decomp(out.bytes(), size, back.view(torch.int16) if n else back.view(torch.int16), n, status.view(torch.int32))
    torch.cuda.synchronize()
    assert int(status.view(torch.int32).item()) == 0
    if n:
        got = to_host(back.view(torch.bfloat16))
        assert np.array_equal(got, x), first_mismatch(got, x)
        back.check("decoded output")
    status.check("status")


def test_scoped_compress_writes_nothing_past_the_stream():
    n = 10 * B + 77
    x = inputs.normal_bf16("test", 9700, n, 1e-3)
    src = guarded_from(x)
    out = Guarded(hc.hc_compress_bound_bf16(n))
    nbytes = Guarded(8)
    ws = Guarded(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_SCOPED, n, 1))
    for group in (1, 3, 0):
        hc.hc_compress_bf16_scoped(src.view(torch.int16), n, out.bytes(), nbytes.view(torch.int64), group,
                                   ws.bytes())
        torch.cuda.synchronize()
        size = int(nbytes.view(torch.int64).item())
        want = oracle.compress_scoped(x, group)
        assert out.bytes()[:size].cpu().numpy().tobytes() == want, f"group {group}"
        out.check(f"scoped stream (group {group})", valid=size)
        nbytes.check("byte count")
        ws.check("scoped workspace")
        out.bytes().fill_(FILL)


def test_corrupt_stream_zeroes_only_the_output():
    n = 4 * B + 9
    x = inputs.normal_bf16("test", 9800, n, 0.02)
    stream = bytearray(oracle.compress(x))
    stream[40 + 8 * 2] ^= 0x10   # an offset of the table: the stream is corrupt
    src = Guarded(len(stream))
    src.bytes().copy_(torch.frombuffer(stream, dtype=torch.uint8))
    back = Guarded(2 * n)
    status = Guarded(4)
    hc.hc_decompress_bf16(src.bytes(), len(stream), back.view(torch.int16), n, status.view(torch.int32))
    torch.cuda.synchronize()
    assert int(status.view(torch.int32).item()) == hc.HC_ERR_CORRUPT_STREAM
    assert not back.bytes().any().item(), "a corrupt stream leaves the whole output zero"
    back.check("decoded output of a corrupt stream")
    status.check("status")


@pytest.mark.parametrize("chain_max", ["0", str(1 << 40)], ids=["steps", "one_launch"])
@pytest.mark.parametrize("R,n", [(4, 40 * B + 123), (3, 3 * B + 5), (8, 16 * B)])
def test_compressed_allreduce_writes_nothing_outside(monkeypatch, chain_max, R, n):
    monkeypatch.setenv("HC_CHAIN_MAX_BYTES", chain_max)
    xs = [inputs.normal_bf16("test", 9900 + r, n, 1e-3) for r in range(R)]
    send = [guarded_from(x) for x in xs]
    recv = [Guarded(2 * n) for _ in range(R)]
    ws = Guarded(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R))
    wire = Guarded(8)
    hc.hc_compressed_allreduce([s.view(torch.bfloat16) for s in send], [r.view(torch.bfloat16) for r in recv], n,
                               ws.bytes(), wire.view(torch.int64))
    torch.cuda.synchronize()
    ref, ref_wire = oracle.compressed_allreduce(xs, chunk=oracle.chunk_elems(n, B))
    for r in range(R):
        got = to_host(recv[r].view(torch.bfloat16))
        assert np.array_equal(got, ref[r]), f"rank {r}: {first_mismatch(got, ref[r])}"
        recv[r].check(f"recvbufs[{r}]")
        send[r].check(f"sendbufs[{r}]")
    assert int(wire.view(torch.int64).item()) == ref_wire
    ws.check("compressed-ring workspace")
    wire.check("wire byte count")
