"""The three-round baseline (hc_compress_bf16_staged: blocks into temporary
slots, a prefix of the sizes, a coalescing copy -- the design "CCCL:
In-GPU Compression-Coupled Collective Communication", section 4.4 replaces)
writes the same HCZ1 bytes as the oracle and as the single-round encoder."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu
B = 16384


def staged(d_in: torch.Tensor, n: int):
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.full((hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_STAGED, n, 1),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    hc.hc_compress_bf16_staged(d_in, n, out, nbytes, ws)
    torch.cuda.synchronize()
    size = int(nbytes.item())
    return to_host(out)[:size]


@pytest.mark.parametrize("n", [0, 1, 9, B - 1, B, B + 1, 3 * B + 77, 1024 * B + 5, 1500 * B])
def test_staged_matches_oracle(n):
    print(f"staged n={n}", flush=True)
    v = inputs.codec_inputs(n)["activations"] if n else np.zeros(0, np.uint16)
    d = to_dev(v) if n else torch.empty(8, dtype=torch.bfloat16, device="cuda")
    got = staged(d, n)
    want = np.frombuffer(oracle.compress(v), np.uint8)
    assert got.size == want.size and np.array_equal(got, want), first_mismatch(got, want)


def test_staged_equals_single_round_full_size():
    """2^28 bf16 weights: byte-identical to hc_compress_bf16 (whose stream the
    codec tests compare with the oracle's)."""
    n = 1 << 28
    x = inputs.normal_bf16_cuda("codec", 0, n, 0.02)
    a = staged(x, n)
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    hc.hc_compress_bf16(x, n, out, nb, ws)
    torch.cuda.synchronize()
    b = to_host(out)[:int(nb.item())]
    assert a.size == b.size and np.array_equal(a, b), first_mismatch(a, b)
