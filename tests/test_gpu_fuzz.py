"""Both decoders against the oracle's on damaged streams: for every input the
GPU decoder and the oracle's decoder must agree -- both reject it (status
HC_ERR_CORRUPT_STREAM, output all zero) or both accept it with the same
output.  A flipped bit inside a code or a plane usually yields another valid
stream; a flipped bit in a header, a length table, an offset or padding must
be rejected by both.

Every damaged stream stays inside its buffer and every read of both decoders
is bounded by the validated header and record lengths, so the damage only
exercises the validation paths."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import to_host

pytestmark = pytest.mark.gpu
B = 16384


def gpu_decode(stream: bytes, n: int, entropy: bool):
    d = torch.from_numpy(np.frombuffer(stream, np.uint8).copy()).to("cuda")
    out = torch.full((max(n, 1),), 1.0, dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    fn = hc.hc_decompress_bf16_entropy if entropy else hc.hc_decompress_bf16
    fn(d, len(stream), out, n, status)
    torch.cuda.synchronize()
    return int(status.item()), to_host(out)[:n]


def damaged(stream: bytes, g: np.random.Generator, hot: list[int]):
    """One damaged copy: a random bit anywhere, a random byte in a hot region
    (headers, tables), or a truncation."""
    b = bytearray(stream)
    kind = g.integers(0, 3)
    if kind == 0:
        i = int(g.integers(0, len(b)))
        b[i] ^= 1 << int(g.integers(0, 8))
    elif kind == 1:
        i = hot[int(g.integers(0, len(hot)))]
        b[i] = int(g.integers(0, 256))
    else:
        b = b[:int(g.integers(16, len(b))) // 16 * 16]
    return bytes(b)


def hot_bytes(stream: bytes, nb: int, coded_table: int):
    """Stream header, offset table, and each record's header and table."""
    hot = list(range(32 + 8 * nb))
    for k in range(nb):
        off = int.from_bytes(stream[32 + 8 * k:40 + 8 * k], "little")
        hot += list(range(off, off + 16 + coded_table))
    return [h for h in hot if h < len(stream)]


@pytest.mark.parametrize("entropy", [False, True])
def test_damaged_streams_agree_with_oracle(entropy):
    n = 3 * B + 1000
    v = inputs.codec_inputs(n)["weights"]
    stream = oracle.hce_compress(v) if entropy else oracle.compress(v)
    ref_decode = oracle.hce_decompress if entropy else oracle.decompress
    nb = -(-n // B)
    hot = hot_bytes(stream, nb, 128 if entropy else 16)
    g = np.random.default_rng(2026 + entropy)
    rejected = accepted = 0
    for k in range(150):
        bad = damaged(stream, g, hot)
        rs, rout = ref_decode(bad, n)
        gs, gout = gpu_decode(bad, n, entropy)
        if rs != 0:
            assert gs == hc.HC_ERR_CORRUPT_STREAM and not gout.any(), f"case {k}: oracle rejects, GPU status {gs}"
            rejected += 1
        else:
            assert gs == 0 and np.array_equal(gout, rout), f"case {k}: oracle accepts, GPU status {gs}"
            accepted += 1
    print(f"entropy={entropy}: {rejected} rejected, {accepted} accepted by both")
    assert rejected > 30 and accepted > 10
