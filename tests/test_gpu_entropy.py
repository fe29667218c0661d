"""GPU parity of the entropy-coded variant (hc_compress_bf16_entropy /
hc_decompress_bf16_entropy, HCE1) against the oracle: the GPU stream equals
the oracle's byte for byte, the GPU decoder restores the input bit for bit
from the oracle's stream, and both reject the same corrupt streams.

"CCCL: In-GPU Compression-Coupled Collective Communication", sections 4.1
and 6.5; Huffman codes, canonical form of RFC 1951 section 3.2.2."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu
B = 16384
WORDS_OFF = 16528


def gpu_compress_dev(d_in: torch.Tensor, n: int):
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.full((hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_ENTROPY, n, 1),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    hc.hc_compress_bf16_entropy(d_in, n, out, nbytes, ws)
    torch.cuda.synchronize()
    return out, int(nbytes.item())


def gpu_decompress(stream_dev: torch.Tensor, in_bytes: int, n: int):
    out = torch.full((max(n, 1),), 1.0, dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    hc.hc_decompress_bf16_entropy(stream_dev, in_bytes, out, n, status)
    torch.cuda.synchronize()
    return int(status.item()), to_host(out)[:n]


def check(v: np.ndarray, label: str):
    print(label, flush=True)
    n = v.size
    ref = oracle.hce_compress(v)
    d = to_dev(v) if n else torch.empty(8, dtype=torch.bfloat16, device="cuda")
    out, size = gpu_compress_dev(d, n)
    assert size == len(ref), f"{label}: size {size} != oracle {len(ref)}"
    got = to_host(out)[:size]
    want = np.frombuffer(ref, np.uint8)
    assert np.array_equal(got, want), f"{label}: {first_mismatch(got, want)}"
    st, back = gpu_decompress(out, size, n)
    assert st == 0 and np.array_equal(back, v), f"{label}: status {st} {first_mismatch(back, v)}"
    # the GPU decoder on the oracle's bytes (a separate copy, read to its exact length)
    dref = torch.from_numpy(want.copy()).to("cuda") if size else torch.zeros(16, dtype=torch.uint8, device="cuda")
    st, back = gpu_decompress(dref, size, n)
    assert st == 0 and np.array_equal(back, v), label


@pytest.mark.parametrize("n", [0, 1, 7, B - 1, B, B + 1, 3 * B + 77, 64 * B, 100 * B + 12345])
def test_ragged_sizes(n):
    check(inputs.normal_bf16("test", 900 + n, n, 1e-3), f"n={n}")


@pytest.mark.parametrize("name", ["weights", "activations", "gradients"])
def test_codec_tensors(name):
    check(inputs.codec_inputs(40 * B + 5)[name], name)


def test_bucket():
    check(inputs.bucket_bf16("test", 8, 150 * B + 3), "bucket")


def block_of(exp_of_index, seed):
    g = np.random.default_rng(seed)
    idx = np.arange(B)
    e = np.asarray(exp_of_index(idx), dtype=np.uint16)
    return (g.integers(0, 2, B).astype(np.uint16) << 15) | (e << 7) | g.integers(0, 128, B).astype(np.uint16)


def test_hand_layouts():
    """The oracle's hand-derived layouts: alternating exponents, the word
    order with two 2-bit lanes, and a lane whose last word is mostly padding."""
    check(block_of(lambda i: 127 + (i // 64) % 2, 1), "alternating")

    def order(i):
        j = i % 64
        return np.where(j == 0, 128, np.where(j == 1, 129, 127))
    check(block_of(order, 2), "word order")
    check(block_of(lambda i: np.where(i == 64 * 255 + 2, 128, order(i)), 5), "padding word")


def test_single_exponent_and_raw_blocks():
    g = np.random.default_rng(6)
    single = np.full(B, 0x3F80, np.uint16) | g.integers(0, 128, B).astype(np.uint16)
    uniform = g.integers(0, 1 << 16, B).astype(np.uint16)
    check(np.concatenate([single, uniform, single[:777]]), "single / uniform / tail")


def test_length_limit_path():
    """Exponent counts 8192, 4096, ..., 2, 1, 1 (15 exponents): the Huffman
    depth reaches 14, so the 12-bit limit and its repair run."""
    counts = [1 << k for k in range(13, 0, -1)] + [1, 1]
    assert sum(counts) == B
    e = np.concatenate([np.full(c, 60 + k, np.uint16) for k, c in enumerate(counts)])
    np.random.default_rng(7).shuffle(e)
    c = np.bincount(e, minlength=256).astype(np.uint32)
    assert oracle.huff_lengths(c, 64).max() > 12
    v = (e << 7) | np.random.default_rng(8).integers(0, 128, B).astype(np.uint16)
    check(np.concatenate([v, v[::-1]]), "length limit")


def test_every_bit_pattern():
    pats = np.arange(1 << 16, dtype=np.uint16)
    g = np.random.default_rng(9)
    check(np.concatenate([pats, g.permutation(pats), np.repeat(pats[::256], 256)]), "all patterns")


def test_corrupt_streams_rejected_like_the_oracle():
    def exps(i):
        j = i % 64
        e = np.where(j == 0, 128, np.where(j == 1, 129, 127))
        return np.where(i == 64 * 255 + 2, 128, e)

    v = block_of(exps, 5)
    good = bytearray(oracle.hce_compress(v))
    rec = 48
    n_words = int.from_bytes(good[rec + 8:rec + 12], "little")
    cases = []
    b = bytearray(good); b[0] ^= 1; cases.append(b)
    b = bytearray(good); b[rec + 16 + 63] = (b[rec + 16 + 63] & 0x0F) | (13 << 4); cases.append(b)
    b = bytearray(good); b[rec + 16 + 10] |= 1; cases.append(b)
    b = bytearray(good); b[rec + 2] += 1; b[rec + 16 + 10] |= 1; cases.append(b)
    b = bytearray(good); b[rec + 8] -= 1; cases.append(b)
    b = bytearray(good); b[rec + WORDS_OFF + 4 * (n_words - 1) + 3] |= 0x80; cases.append(b)
    b = bytearray(good); b[rec + 1] = 11; cases.append(b)
    b = bytearray(good); b[rec] = 1; cases.append(b)
    for k, bad in enumerate(cases):
        assert oracle.hce_decompress(bytes(bad), B)[0] == 4
        d = torch.from_numpy(np.frombuffer(bytes(bad), np.uint8).copy()).to("cuda")
        st, back = gpu_decompress(d, len(bad), B)
        assert st == hc.HC_ERR_CORRUPT_STREAM and not back.any(), f"case {k}"
    d = torch.from_numpy(np.frombuffer(bytes(good), np.uint8).copy()).to("cuda")
    st, _ = gpu_decompress(d, len(good) - 16, B)   # truncated
    assert st == hc.HC_ERR_CORRUPT_STREAM


def test_workspace_reuse():
    n = 9 * B + 5
    v = inputs.normal_bf16("test", 31, n, 0.02)
    d = to_dev(v)
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_ENTROPY, n, 1), dtype=torch.uint8, device="cuda")
    ref = oracle.hce_compress(v)
    for _ in range(3):
        hc.hc_compress_bf16_entropy(d, n, out, nb, ws)
        torch.cuda.synchronize()
        assert int(nb.item()) == len(ref) and to_host(out)[:len(ref)].tobytes() == ref


@pytest.mark.parametrize("name", ["weights", "activations"])
def test_full_size(name):
    """2^28 bf16 (the codec workload): the whole stream against the oracle's,
    and the GPU round trip."""
    n = 1 << 28
    print(f"full size {name}", flush=True)
    x = (inputs.normal_bf16_cuda("codec", 0, n, 0.02) if name == "weights"
         else inputs.activation_bf16_cuda("codec", 1, n))
    out, size = gpu_compress_dev(x, n)
    ref = oracle.hce_compress(inputs.host_bits(x))
    assert size == len(ref)
    got = to_host(out)[:size]
    want = np.frombuffer(ref, np.uint8)
    assert np.array_equal(got, want), first_mismatch(got, want)
    del got, want, ref
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    hc.hc_decompress_bf16_entropy(out, size, back, n, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.equal(back.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("k", [2, 3, 63, 64, 65, 80, 200])
def test_exponent_count_boundaries(k):
    """k distinct exponents per block with skewed counts: up to 64 the code
    is built in one wave's registers, above that by the LDS loop."""
    g = np.random.default_rng(100 + k)
    p = 1.0 / np.arange(1, k + 1) ** 1.1
    p /= p.sum()
    blocks = []
    for b in range(3):
        e = g.choice(np.arange(60, 60 + k), size=B, p=p).astype(np.uint16)
        e[:k] = np.arange(60, 60 + k)            # every exponent present
        g.shuffle(e)
        blocks.append((e << 7) | g.integers(0, 128, B).astype(np.uint16))
    v = np.concatenate(blocks)
    assert all(len(np.unique((blk >> 7) & 0xFF)) == k for blk in blocks)
    check(v, f"k={k}")
