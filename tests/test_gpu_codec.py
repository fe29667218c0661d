"""GPU parity of the HCZ1 codec (hc_compress_bf16 / hc_decompress_bf16)
against the oracle: the GPU stream must equal the oracle's stream byte for
byte, and decoding must restore the input bit for bit.

Codec: "CCCL: In-GPU Compression-Coupled Collective Communication", sections
4.1, 4.3, 4.4 and 5 ("Handling data alignment")."""
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu
B = 16384
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_compress(v: np.ndarray):
    n = v.size
    d_in = to_dev(v) if n else torch.empty(8, dtype=torch.bfloat16, device="cuda")
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    hc.hc_compress_bf16(d_in, n, out, nbytes, ws)
    torch.cuda.synchronize()
    size = int(nbytes.item())
    return to_host(out)[:size].tobytes(), out, size


def gpu_decompress(stream_dev: torch.Tensor, in_bytes: int, n: int):
    out = torch.full((max(n, 1),), 1.0, dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    hc.hc_decompress_bf16(stream_dev, in_bytes, out, n, status)
    torch.cuda.synchronize()
    return int(status.item()), to_host(out)[:n]


def check_roundtrip(v: np.ndarray, label: str):
    ref = oracle.compress(v)
    got, dev_stream, size = gpu_compress(v)
    assert size == len(ref), f"{label}: size {size} != oracle {len(ref)}"
    if got != ref:
        a = np.frombuffer(got, np.uint8)
        b = np.frombuffer(ref, np.uint8)
        raise AssertionError(f"{label}: stream differs: {first_mismatch(a, b)}")
    st, back = gpu_decompress(dev_stream, size, v.size)
    assert st == 0, f"{label}: status {st}"
    assert np.array_equal(back, v), f"{label}: {first_mismatch(back, v)}"


def golden_cases():
    from test_oracle_codec import read_examples
    return read_examples()


def test_worked_examples_bit_exact():
    for name, v, _plan, total in golden_cases():
        check_roundtrip(v, name)
        assert len(oracle.compress(v)) == total


@pytest.mark.parametrize("n", [0, 1, 5, 8, 9, B - 1, B, B + 1, 3 * B + 77, 64 * B, 100 * B + 12345])
def test_ragged_sizes_bit_exact(n):
    v = inputs.normal_bf16("test", n, n, 1e-3)
    check_roundtrip(v, f"n={n}")


def test_all_bit_patterns():
    pats = np.arange(1 << 16, dtype=np.uint16)
    check_roundtrip(pats, "consecutive patterns")
    g = np.random.default_rng(5)
    blocks = []
    for k in range(0, pats.size, 1384):
        blk = np.full(B, 0x3F80, np.uint16)
        part = pats[k:k + 1384]
        blk[g.choice(B, part.size, replace=False)] = part
        blocks.append(blk)
    check_roundtrip(np.concatenate(blocks), "patterns inside coded blocks")
    flat = ((np.arange(B) % 256).astype(np.uint16) << 7) | g.integers(0, 128, B).astype(np.uint16)
    check_roundtrip(flat.astype(np.uint16), "raw block")


@pytest.mark.parametrize("kind", ["weights", "activations", "gradients"])
def test_codec_workloads_reduced(kind):
    n = 64 * B + 999
    v = {"weights": lambda: inputs.normal_bf16("codec", 0, n, 0.02),
         "activations": lambda: inputs.activation_bf16("codec", 1, n),
         "gradients": lambda: inputs.normal_bf16("codec", 2, n, 1e-4)}[kind]()
    check_roundtrip(v, kind)


def test_decodes_oracle_streams():
    """The decoder reads streams written by the oracle (not by the GPU encoder)."""
    for seed, sigma in ((1, 0.02), (2, 1.0), (3, 1e-4)):
        v = inputs.normal_bf16("test", 100 + seed, 5 * B + seed, sigma)
        s = oracle.compress(v)
        dev = torch.from_numpy(np.frombuffer(s, np.uint8).copy()).to("cuda")
        st, back = gpu_decompress(dev, len(s), v.size)
        assert st == 0 and np.array_equal(back, v)


def test_corrupt_streams_rejected_like_oracle():
    from test_oracle_codec import build_case, corrupt_cases
    v = build_case("eighth", ["0x3F80", "0x4000"])
    v = np.concatenate([v, v[:100]])
    s = oracle.compress(v)
    for name, bad, nbytes in corrupt_cases(s):
        dev = torch.from_numpy(np.frombuffer(bad, np.uint8).copy()).to("cuda")
        st, out = gpu_decompress(dev, nbytes, v.size)
        ost, oout = oracle.decompress(bad[:nbytes], v.size)
        assert ost == oracle.CORRUPT
        assert st == hc.HC_ERR_CORRUPT_STREAM, name
        assert not out.any(), name
    # wrong element count
    dev = torch.from_numpy(np.frombuffer(s, np.uint8).copy()).to("cuda")
    st, _ = gpu_decompress(dev, len(s), v.size + 1)
    assert st == hc.HC_ERR_CORRUPT_STREAM
    # an empty stream with a damaged header
    e = bytearray(oracle.compress(np.zeros(0, np.uint16)))
    e[0] ^= 1
    dev = torch.from_numpy(np.frombuffer(bytes(e), np.uint8).copy()).to("cuda")
    st, _ = gpu_decompress(dev, len(e), 0)
    assert st == hc.HC_ERR_CORRUPT_STREAM


@pytest.mark.parametrize("kind", ["weights", "activations", "gradients"])
def test_codec_full_size(kind):
    """The codec workload's three 2^28 bf16 tensors (weights N(0, 0.02),
    activations, gradients N(0, 1e-4)): GPU stream == oracle stream; round trip."""
    n = 1 << 28
    t = {"weights": lambda: inputs.normal_bf16_cuda("codec", 0, n, 0.02),
         "activations": lambda: inputs.activation_bf16_cuda("codec", 1, n),
         "gradients": lambda: inputs.normal_bf16_cuda("codec", 2, n, 1e-4)}[kind]()
    v = inputs.host_bits(t)
    del t
    check_roundtrip(v, f"{kind} 2^28")
    torch.cuda.empty_cache()


def test_back_to_back_calls_place_every_record():
    """Block j is workgroup j and its look-back waits only on lower-indexed
    blocks: 200 back-to-back calls on 2^24 elements (1,024 blocks, more than
    fit on the GPU at once), on two encoders sharing the writer, each give the
    full stream (a look-back that gave up would report 0 bytes) with the same
    bytes as the oracle's."""
    n = 1 << 24
    g = np.random.default_rng(2024)
    v = inputs.f32_to_bf16_bits((g.standard_normal(n) * 0.02).astype(np.float32))
    ref = np.frombuffer(oracle.compress(v), np.uint8)
    d_in = to_dev(v)
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(200, dtype=torch.int64, device="cuda")
    for k in range(200):
        hc.hc_compress_bf16(d_in, n, out, sizes[k:k + 1], ws)
    torch.cuda.synchronize()
    assert torch.all(sizes == ref.size).item(), sizes.unique().tolist()
    assert np.array_equal(to_host(out)[:ref.size], ref)
    hsizes = torch.zeros(100, dtype=torch.int64, device="cuda")
    hws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_ENTROPY, n, 1), dtype=torch.uint8, device="cuda")
    hout = torch.empty(hc.hc_compress_bound_bf16(n), dtype=torch.uint8, device="cuda")
    for k in range(100):
        hc.hc_compress_bf16_entropy(d_in, n, hout, hsizes[k:k + 1], hws)
    torch.cuda.synchronize()
    href = np.frombuffer(oracle.hce_compress(v), np.uint8)
    assert torch.all(hsizes == href.size).item(), hsizes.unique().tolist()
    assert np.array_equal(to_host(hout)[:href.size], href)
