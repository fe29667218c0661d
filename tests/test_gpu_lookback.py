"""The bounded look-back wait of the single-pass stream encoders, forced to
give up from the host (HC_LOOKBACK_SPIN_LIMIT, read at every call).

A block whose wait for its predecessors' sizes runs past its bound publishes
poison, writes nothing and sets the error word; the last block waits (also
bounded) until every other block has ended its walk before it reads that
word.  So a call either reports a zero-byte stream or writes exactly the
oracle's stream -- never a stream with a missing record reported as valid.
Every kernel exits normally: all waits are bounded."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs

pytestmark = pytest.mark.gpu
B = 16384


def encoders():
    def ws_call(fn, op):
        def call(x, n, out, nb):
            ws = torch.empty(hc.hc_workspace_bytes(op, n, 1), dtype=torch.uint8, device="cuda")
            fn(x, n, out, nb, ws)
        return call

    def scoped(x, n, out, nb):
        ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_SCOPED, n, 1), dtype=torch.uint8, device="cuda")
        hc.hc_compress_bf16_scoped(x, n, out, nb, 1, ws)

    return {
        "hcz1": (ws_call(hc.hc_compress_bf16, hc.HC_OP_COMPRESS), oracle.compress),
        "noalloc": (lambda x, n, out, nb: hc.hc_compress_bf16_noalloc(x, n, out, nb), oracle.compress),
        "scoped": (scoped, lambda v: oracle.compress_scoped(v, 1)),
        "hce1": (ws_call(hc.hc_compress_bf16_entropy, hc.HC_OP_COMPRESS_ENTROPY), oracle.hce_compress),
    }


@pytest.mark.parametrize("coder", ["hcz1", "noalloc", "scoped", "hce1"])
@pytest.mark.parametrize("limit", ["1", "3", "64"])
def test_gave_up_walks_report_no_stream(coder, limit, monkeypatch):
    call, ref = encoders()[coder]
    n = 512 * B + 77
    x = inputs.normal_bf16_cuda("test", 4400, n, 0.02).view(torch.int16)
    want = ref(x.cpu().numpy().view(np.uint16))
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    monkeypatch.setenv("HC_LOOKBACK_SPIN_LIMIT", limit)
    outcomes = {"none": 0, "exact": 0}
    for _ in range(6):
        out.fill_(0xEE)
        call(x, n, out, nb)
        torch.cuda.synchronize()
        size = int(nb.item())
        if size == 0:
            outcomes["none"] += 1
        else:
            assert size == len(want), f"limit {limit}: a stream of {size} bytes reported, the oracle's is {len(want)}"
            assert out[:size].cpu().numpy().tobytes() == want, f"limit {limit}: reported stream differs"
            outcomes["exact"] += 1
    print(f"{coder} spin limit {limit}: {outcomes}", flush=True)
    # the default bound again: the exact stream
    monkeypatch.delenv("HC_LOOKBACK_SPIN_LIMIT")
    call(x, n, out, nb)
    torch.cuda.synchronize()
    size = int(nb.item())
    assert size == len(want) and out[:size].cpu().numpy().tobytes() == want


def test_invalid_limit_values_keep_the_default(monkeypatch):
    n = 64 * B
    x = inputs.normal_bf16_cuda("test", 4401, n, 1e-4).view(torch.int16)
    want = oracle.compress(x.cpu().numpy().view(np.uint16))
    out = torch.empty(hc.hc_compress_bound_bf16(n), dtype=torch.uint8, device="cuda")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    for bad in ("0", "-3", "abc", "", "99999999999"):
        monkeypatch.setenv("HC_LOOKBACK_SPIN_LIMIT", bad)
        hc.hc_compress_bf16(x, n, out, nb, ws)
        torch.cuda.synchronize()
        assert out[:int(nb.item())].cpu().numpy().tobytes() == want, bad
