"""Sizes past 2^32 elements (8 GB of bf16 per buffer): element indices, slice
offsets and record offsets are 64-bit everywhere.

- Ring allreduce, R=2 ranks of 2^32 + 36901 bf16 each: slice 1 starts past
  2^31 and ends past 2^32.  Both ranks must be identical, and sampled indices
  (random ones plus every boundary at 2^31, 2^32 and the slice edge) must
  equal the oracle's ring fold.
- Codec, 2^32 + 36901 bf16: compress then decompress gives the input back bit
  for bit, and the records of the blocks on either side of 2^32 and of the
  partial last block equal the oracle's records for the same elements.

Inputs come from torch's seeded generator on the device and are copied to
the host for the oracle (16 GB of host memory)."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc

pytestmark = pytest.mark.gpu
B = 16384
N = (1 << 32) + 2 * B + 4133


def bf16_input(seed: int, n: int, scale: float) -> torch.Tensor:
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    step = 1 << 28
    for lo in range(0, n, step):  # in pieces: fp32 staging stays at 1 GB
        hi = min(n, lo + step)
        out[lo:hi] = (torch.randn(hi - lo, generator=g, device="cuda") * scale).to(torch.bfloat16)
    return out


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_allreduce_past_2e32_elements():
    R, n = 2, N
    L = -(-n // R)
    print(f"allreduce R={R} n={n} L={L}", flush=True)
    xs = [bf16_input(100 + r, n, 1e-3) for r in range(R)]
    outs = [torch.empty_like(x) for x in xs]
    hc.hc_allreduce(xs, outs)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "ranks differ"
    g = np.random.default_rng(7)
    edges = [0, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, L - 1, L, L + 1, (1 << 32) - 1, 1 << 32, (1 << 32) + 1, n - 1]
    idx = np.unique(np.concatenate([g.integers(0, n, 1 << 16, dtype=np.uint64), np.array(edges, dtype=np.uint64)]))
    got = host_bits(outs[0][torch.from_numpy(idx.astype(np.int64)).to("cuda")])
    host = [host_bits(x) for x in xs]
    want = oracle.allreduce_fold_at(host, idx)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at index {int(idx[bad[0]])}"


def test_codec_round_trip_past_2e32_elements():
    n = N
    nb = -(-n // B)
    print(f"codec n={n} blocks={nb}", flush=True)
    x = bf16_input(300, n, 0.02)
    cap = hc.hc_compress_bound_bf16(n)
    stream = torch.empty(cap, dtype=torch.uint8, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    hc.hc_compress_bf16(x, n, stream, size, ws)
    torch.cuda.synchronize()
    m = int(size.item())
    assert 0 < m <= cap
    back = torch.empty_like(x)
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    hc.hc_decompress_bf16(stream, m, back, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(back.view(torch.int16), x.view(torch.int16)), "round trip differs"
    offs = stream[32:32 + 8 * nb].cpu().numpy().view(np.uint64)
    xh = host_bits(x)
    for k in ((1 << 32) // B - 1, (1 << 32) // B, nb - 1):
        lo, hi = k * B, min(n, (k + 1) * B)
        ref = oracle.compress(xh[lo:hi])
        r_off = int.from_bytes(ref[32:40], "little")
        r_total = int.from_bytes(ref[24:32], "little")
        end = int(offs[k + 1]) if k + 1 < nb else m
        got = stream[int(offs[k]):end].cpu().numpy().tobytes()
        assert got == ref[r_off:r_total], f"record of block {k} differs"
