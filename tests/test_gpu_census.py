"""CU placement of the CU-budget streams (the contention workload's side
stream).  "HOCCL: Offloading Collective Communication from GPU Cores to
Accelerate Distributed Training" (section 2) measures the share of cores a
collective holds while compute runs; that share is the stream's CU budget
only if the budget really confines the reduce-scatter to k CUs.  A census
kernel records the XCD and CU of every workgroup of a launch that
oversubscribes the stream, so every allowed CU is used."""
import collections

import pytest
import torch

from collective_communication_amd import binding as hc

pytestmark = pytest.mark.gpu


def census(handle, n_workgroups):
    st = torch.cuda.ExternalStream(handle) if handle else None
    ids = hc.hc_cu_census(n_workgroups, 50, stream=st)
    rows = [tuple(r) for r in ids.tolist()]
    return set(rows), collections.Counter(x for x, _ in rows)


def n_cu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def test_default_stream_spans_every_cu():
    cus, per_xcc = census(None, n_cu() * 40)
    assert len(cus) == n_cu()
    assert len(per_xcc) == 8 and len({c for c in per_xcc.values()}) == 1, per_xcc


@pytest.mark.parametrize("k", [8, 16, 32, 64])
def test_cu_budget_stream_holds_exactly_k_cus_spread_over_xcds(k):
    h = hc.hc_stream_create_cu_budget(k)
    try:
        cus, _ = census(h, 64 * k)   # 64 one-wave workgroups per allowed CU: more than fit at once
    finally:
        hc.hc_stream_destroy(h)
    assert len(cus) == k, sorted(cus)
    per_xcc = collections.Counter(x for x, _ in cus)
    assert sorted(per_xcc) == list(range(8)) and set(per_xcc.values()) == {k // 8}, per_xcc


@pytest.mark.parametrize("k", [8, 32])
def test_budget_and_its_complement_share_no_cu(k):
    ncu = n_cu()
    a = hc.hc_stream_create_cu_budget(k)
    b = hc.hc_stream_create_cu_range(k, ncu - k)
    try:
        ca, _ = census(a, 64 * k)
        cb, _ = census(b, 40 * ncu)
    finally:
        hc.hc_stream_destroy(a)
        hc.hc_stream_destroy(b)
    assert len(ca) == k and len(cb) == ncu - k
    assert not (ca & cb) and len(ca | cb) == ncu


def test_reduce_scatter_kernels_run_inside_the_budget():
    """The reduce-scatter's persistent grid on a k-CU stream leaves the other
    CUs free: a census launched on the complement right behind it on another
    stream starts while the reduce-scatter still runs (both finish), and the
    census sees only complement CUs."""
    R, L, k = 8, 1 << 22, 8
    send = [torch.randn(R * L, device="cuda").to(torch.bfloat16) for _ in range(R)]
    recv = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, R * L, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    a = hc.hc_stream_create_cu_budget(k)
    b = hc.hc_stream_create_cu_range(k, n_cu() - k)
    try:
        sa = torch.cuda.ExternalStream(a)
        hc.hc_reduce_scatter(send, recv, L, ws, cu_budget=k, stream=sa)
        cb, _ = census(b, 20 * n_cu())
        sa.synchronize()
        ca, _ = census(a, 64 * k)
    finally:
        hc.hc_stream_destroy(a)
        hc.hc_stream_destroy(b)
    assert not (ca & cb) and len(cb) == n_cu() - k
