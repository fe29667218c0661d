"""GPU parity of the bf16 allreduce with fp32 partials (one final rounding)
against the oracle's fp32-carry fold, bit for bit: ranks 1..8 and 16, sizes
with short, empty and unaligned slices (the element-wise path), chunk
fractions, in place, the copy-engine all-gather, a workspace full of garbage,
and the full R=8 x 2^26 workload; plus the hand-derived case in which one
rounding keeps what per-hop rounding drops."""
import numpy as np
import pytest
import torch

import oracle
from collective_communication_amd import binding as hc
from collective_communication_amd import inputs
from hc_util import copy_engine_or_unsupported, first_mismatch, to_dev, to_host

pytestmark = pytest.mark.gpu


def rand_bf16(R, n, seed, scale=1e-3):
    g = np.random.default_rng(seed)
    return [inputs.f32_to_bf16_bits((g.standard_normal(n) * scale).astype(np.float32)) for _ in range(R)]


def workspace(n, R, fill=None):
    need = hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, n, R, hc.HC_BF16)
    if need == 0:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    if fill is not None:
        ws.fill_(fill)
    return ws


def run(xs, *, inplace=False, fill=None, **kw):
    R, n = len(xs), xs[0].size
    send = [to_dev(x) for x in xs]
    recv = send if inplace else [torch.empty_like(s) for s in send]
    hc.hc_allreduce_bf16_f32carry(send, recv, n, workspace(n, R, fill), **kw)
    torch.cuda.synchronize()
    return [to_host(r) for r in recv]


def check(xs, got, label):
    ref = oracle.allreduce_fold_f32carry(xs)
    for r in range(len(xs)):
        assert np.array_equal(got[r], ref[r]), f"{label} rank {r}: {first_mismatch(got[r], ref[r])}"


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 16])
def test_matches_oracle(R):
    for n in (1, 7, 1000, 8 * 4096 + 3, 3 * 16384 + 17, 1 << 16):
        print(f"f32carry R={R} n={n}", flush=True)
        xs = rand_bf16(R, n, 1000 * R + n)
        check(xs, run(xs), f"R={R} n={n}")


@pytest.mark.parametrize("frac", [0.001, 0.05, 1.0])
def test_chunk_fraction_changes_no_value(frac):
    xs = rand_bf16(8, 100003, 77)
    check(xs, run(xs, chunk_fraction=frac), f"chunk fraction {frac}")


def test_in_place_copy_engine_and_garbage_workspace():
    xs = rand_bf16(4, 65536 + 9, 91)
    check(xs, run(xs, inplace=True), "in place")
    out = []
    if copy_engine_or_unsupported(lambda: out.append(run(xs, copy_engine=1))):
        check(xs, out[0], "copy engine")
    check(xs, run(xs, fill=0xFF), "workspace of 0xFF bytes")   # NaN patterns in every slot


@pytest.mark.parametrize("budget", [8, 32])
def test_cu_budget_grid(budget):
    # A persistent grid of 8 workgroups per budgeted CU (64 or 256) walks the
    # ~320 tiles of every step in a grid-stride loop.
    xs = rand_bf16(8, 8 * 4096 * 40 + 11, 300 + budget)
    check(xs, run(xs, cu_budget=budget), f"cu_budget {budget}")


def test_one_rounding_against_per_hop():
    # n = R = 4: element j lies in slice j; rank j+1 holds 1.0, the others
    # 2^-8.  One rounding gives 1 + 2^-6 (0x3F82), per-hop rounding 1.0.
    R = 4
    xs = [np.array([0x3F80 if r == (j + 1) % R else 0x3B80 for j in range(R)], dtype=np.uint16) for r in range(R)]
    got = run(xs)
    assert all(g.tolist() == [0x3F82] * R for g in got)
    send = [to_dev(x) for x in xs]
    recv = [torch.empty_like(s) for s in send]
    hc.hc_allreduce(send, recv)
    torch.cuda.synchronize()
    assert to_host(recv[0]).tolist() == [0x3F80] * R


def test_full_workload():
    R, n = 8, 1 << 26
    send = inputs.ring_inputs_cuda("ring_bf16", R, n)
    recv = [torch.empty_like(s) for s in send]
    hc.hc_allreduce_bf16_f32carry(send, recv, n, workspace(n, R))
    torch.cuda.synchronize()
    for r in range(1, R):
        assert torch.equal(recv[r].view(torch.int16), recv[0].view(torch.int16)), f"rank {r} differs"
    xs = [inputs.host_bits(t) for t in send]
    ref = oracle.allreduce_fold_f32carry(xs)[0]
    got = to_host(recv[0])
    assert np.array_equal(got, ref), first_mismatch(got, ref)
