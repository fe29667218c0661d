"""Host-side checks of libhc (no GPU needed): it loads, exports every symbol
include/hc.h declares, and its host logic (chunking, the ring task list, the
compression bound, workspace sizes, argument checks) agrees with the oracle
and the header's contract.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "collective_communication_amd", "libhc.so")


@pytest.fixture(scope="module")
def hc():
    if not os.path.exists(LIB):
        pytest.skip("libhc.so not built")
    from collective_communication_amd import binding
    return binding


def header_symbols():
    text = open(os.path.join(ROOT, "include", "hc.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hc_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(hc):
    syms = header_symbols()
    assert len(syms) >= 15
    lib = ctypes.CDLL(LIB)
    for s in syms:
        assert hasattr(lib, s), f"libhc.so does not export {s}"
    assert sorted(hc.EXPORTED) == syms


def test_chunk_matches_oracle(hc):
    for n in (1, 5, 1 << 20, 1 << 25, 1 << 26, 1 << 28, 123457):
        for align in (1024, 16384):
            assert hc.hc_chunk_elems(n, 0.01, align) == oracle.chunk_elems(n, align)


@pytest.mark.parametrize("R,n", [(1, 10), (2, 7), (4, 1 << 20), (8, 1 << 26), (5, 1031), (8, 3)])
def test_task_list_matches_oracle(hc, R, n):
    chunk = oracle.chunk_elems(n)
    ours = np.array(hc.hc_ring_tasks(R, n, chunk), dtype=np.uint64).reshape(-1, 8)
    ref = oracle.ring_tasks(R, n, chunk)
    assert ours.shape[0] == ref.size
    for k, f in enumerate(["src", "dst", "step", "chunk", "op", "slice", "off", "len"]):
        np.testing.assert_array_equal(ours[:, k], ref[f].astype(np.uint64))


def test_compress_bound_matches_oracle(hc):
    for n in (0, 1, 5, 16383, 16384, 16385, 1 << 20, (1 << 28) + 7):
        assert hc.hc_compress_bound_bf16(n) == oracle.compress_bound(n)


def test_workspace_sizes(hc):
    assert hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, 8 * 1000, 8, hc.HC_BF16) == 2 * 8000 * 2
    assert hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, 7, 2, hc.HC_F32) == 0  # 7 % 2 != 0
    assert hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, 1 << 20, 1) > 0
    # the three-round baseline holds one 32,784-byte slot per block
    assert hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_STAGED, 1 << 20, 1) >= 64 * 32784
    # the table-scope encoder also holds per-block histograms and escape counts
    assert hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_SCOPED, 1 << 20, 1) > \
        hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, 1 << 20, 1) + 64 * 256 * 2
    assert hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, 1 << 20, 8, hc.HC_BF16) > 0
    assert hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, 1 << 20, 8, hc.HC_F32) == 0
    assert hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, 64, 0, hc.HC_F32) == 0
    # fp32-carry allreduce: two fp32 slots of ceil(count/R) rounded up to 64 per rank; none for R <= 2
    assert hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, 1000, 8, hc.HC_BF16) == 8 * 2 * 128 * 4
    assert hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, 1 << 26, 8, hc.HC_BF16) == 2 * (1 << 26) * 4
    assert hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, 1000, 2, hc.HC_BF16) == 0
    assert hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, 1000, 8, hc.HC_F32) == 0


def _raw(hc):
    return hc.load()


def test_argument_errors_before_any_launch(hc):
    L = _raw(hc)
    PP = ctypes.POINTER(ctypes.c_void_p)

    def arr(vals):
        a = (ctypes.c_void_p * len(vals))(*vals)
        return ctypes.cast(a, PP), a

    good, _k1 = arr([0x100000, 0x200000])
    good2, _k2 = arr([0x300000, 0x400000])
    mis, _k3 = arr([0x100002, 0x200000])
    null, _k4 = arr([0x100000, 0])
    E = hc.HC_ERR_INVALID_ARGUMENT
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 0, None, None) == E          # R = 0
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 65, None, None) == E         # R > 64
    assert L.hc_allreduce(good, good2, 16, 7, 2, None, None) == E                  # dtype
    assert L.hc_allreduce(mis, good2, 16, hc.HC_F32, 2, None, None) == E           # alignment
    assert L.hc_allreduce(null, good2, 16, hc.HC_F32, 2, None, None) == E          # NULL
    assert L.hc_allreduce(None, good2, 16, hc.HC_F32, 2, None, None) == E
    assert b"aligned" in L.hc_last_error() or b"NULL" in L.hc_last_error()
    # overlapping outputs
    ov, _k5 = arr([0x300000, 0x300010])
    assert L.hc_allreduce(good, ov, 16, hc.HC_F32, 2, None, None) == E
    # output overlapping another rank's input
    cross, _k6 = arr([0x200000, 0x400000])
    assert L.hc_allreduce(good, cross, 16, hc.HC_F32, 2, None, None) == E
    # bad options
    o = hc.hc_opts_t(1.5, 0, 0, None)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    o = hc.hc_opts_t(0.01, -1, 0, None)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    o = hc.hc_opts_t(0.01, 0, -3, None)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    # too few step events for 2(R-1) = 2 steps + 1
    evs = (ctypes.c_void_p * 2)(0x10, 0x20)
    o = hc.hc_opts_t(0.0, 0, 2, ctypes.cast(evs, ctypes.c_void_p))
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    # kernel-stamped steps need two events per step: 3 serve boundaries, not stamps
    evs3 = (ctypes.c_void_p * 3)(0x10, 0x20, 0x30)
    o = hc.hc_opts_t(0.0, 0, 3, ctypes.cast(evs3, ctypes.c_void_p), 0, 1)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    assert b"n_step_events 3 < 4" in L.hc_last_error()
    # copy_engine must be 0 or 1, step_event_mode 0 or 1
    o = hc.hc_opts_t(0.0, 0, 0, None, 2, 0)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    assert b"copy_engine" in L.hc_last_error()
    o = hc.hc_opts_t(0.0, 0, 0, None, 0, 2)
    assert L.hc_allreduce(good, good2, 16, hc.HC_F32, 2, ctypes.byref(o), None) == E
    assert b"step_event_mode" in L.hc_last_error()
    # the compressed allreduce decodes in its all-gather: no copy engine
    o = hc.hc_opts_t(0.0, 0, 0, None, 1, 0)
    assert L.hc_compressed_allreduce(good, good2, 1 << 16, 2, 0x900000, 1 << 30, None, ctypes.byref(o),
                                     None) == hc.HC_ERR_UNSUPPORTED
    # fused allreduce + SGD: lr must be finite; grads and weights may not overlap
    assert L.hc_allreduce_sgd(good, good2, 16, hc.HC_F32, 2, float("nan"), None, None) == E
    assert L.hc_allreduce_sgd(good, good2, 16, hc.HC_F32, 2, float("inf"), None, None) == E
    assert L.hc_allreduce_sgd(good, good, 16, hc.HC_F32, 2, 0.1, None, None) == E
    assert b"overlap" in L.hc_last_error()
    assert L.hc_allreduce_sgd(null, good2, 16, hc.HC_F32, 2, 0.1, None, None) == E
    assert L.hc_allreduce_sgd(good, good2, 0, hc.HC_F32, 2, 0.1, None, None) == hc.HC_SUCCESS
    # count 0 is a no-op success
    assert L.hc_allreduce(good, good2, 0, hc.HC_F32, 2, None, None) == hc.HC_SUCCESS
    # reduce-scatter: missing / small / misaligned workspace
    assert L.hc_reduce_scatter(good, good2, 16, hc.HC_F32, 2, None, 0, None, None) == E
    assert L.hc_reduce_scatter(good, good2, 16, hc.HC_F32, 2, 0x900000, 16, None, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_reduce_scatter(good, good2, 16, hc.HC_F32, 2, 0x900008, 1 << 20, None, None) == E
    # compress: capacity below the bound
    assert L.hc_compress_bf16(0x100000, 1000, 0x200000, 100, 0x300000, 0x400000, 1 << 20, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_compress_bf16(0x100000, 1000, 0x200000, 1 << 20, None, 0x400000, 1 << 20, None) == E
    # scoped compress: the plain encoder's workspace is too small, capacity below the bound
    n = 1 << 20
    small = hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1)
    assert L.hc_compress_bf16_scoped(0x10000000, n, 0x20000000, 1 << 24, 0x30000000, 0, 0x40000000, small,
                                     None) == hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_compress_bf16_scoped(0x10000000, n, 0x20000000, 100, 0x30000000, 4, 0x40000000, 1 << 26,
                                     None) == hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_compress_bf16_scoped(None, n, 0x20000000, 1 << 24, 0x30000000, 4, 0x40000000, 1 << 26,
                                     None) == E
    # allocation-free compress: n beyond the static scratch, capacity, NULL and alignment, all before any
    # device call
    big = (1 << 31) + 1
    assert L.hc_compress_bf16_noalloc(0x100000, big, 0x200000, 1 << 40, 0x300000, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert b"static scratch" in L.hc_last_error()
    assert L.hc_compress_bf16_noalloc(0x100000, 1000, 0x200000, 100, 0x300000, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_compress_bf16_noalloc(0x100000, 1000, 0x200000, 1 << 20, None, None) == E
    assert L.hc_compress_bf16_noalloc(None, 1000, 0x200000, 1 << 20, 0x300000, None) == E
    assert L.hc_compress_bf16_noalloc(0x100008, 1000, 0x200000, 1 << 20, 0x300000, None) == E
    assert L.hc_compress_bf16_noalloc(0x100000, 1000, 0x100100, 1 << 20, 0x300000, None) == E   # overlap
    # decompress: status word is required
    assert L.hc_decompress_bf16(0x100000, 1000, 0x200000, 100, None, None) == E
    # compressed allreduce: workspace too small
    assert L.hc_compressed_allreduce(good, good2, 1 << 16, 2, 0x900000, 16, None, None, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    # fp32-carry allreduce: workspace needed from 3 ranks on, aligned, large enough, apart from the buffers
    three, _k7 = arr([0x100000, 0x200000, 0x300000])
    three_out, _k8 = arr([0x400000, 0x500000, 0x600000])
    need = hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, 16, 3, hc.HC_BF16)
    assert L.hc_allreduce_bf16_f32carry(three, three_out, 16, 3, None, 0, None, None) == E
    assert L.hc_allreduce_bf16_f32carry(three, three_out, 16, 3, 0x900000, need - 1, None, None) == \
        hc.HC_ERR_INSUFFICIENT_CAPACITY
    assert L.hc_allreduce_bf16_f32carry(three, three_out, 16, 3, 0x900008, need, None, None) == E
    assert L.hc_allreduce_bf16_f32carry(three, three_out, 16, 3, 0x400000, need, None, None) == E
    assert b"overlaps" in L.hc_last_error()
    odd, _k9 = arr([0x100001, 0x200000])   # bf16 pointers need 2-byte alignment
    assert L.hc_allreduce_bf16_f32carry(odd, good2, 16, 2, None, 0, None, None) == E
    assert L.hc_allreduce_bf16_f32carry(good, good2, 16, 65, None, 0, None, None) == E
    assert L.hc_allreduce_bf16_f32carry(good, good2, 0, 2, None, 0, None, None) == hc.HC_SUCCESS
    # CU-budget stream: k out of range (no device is touched for k < 1)
    s = ctypes.c_void_p(0)
    assert L.hc_stream_create_cu_budget(0, ctypes.byref(s)) != hc.HC_SUCCESS
    assert L.hc_stream_create_cu_range(0, 0, ctypes.byref(s)) == E
    assert L.hc_stream_create_cu_range(-1, 8, ctypes.byref(s)) == E
    assert L.hc_stream_create_cu_range(0, 8, None) == E
    # CU census: arguments checked before any launch
    assert L.hc_cu_census(None, 8, 10, None) == E
    assert L.hc_cu_census(0x100002, 8, 10, None) == E
    assert L.hc_cu_census(0x100000, 0, 10, None) == E
    assert L.hc_cu_census(0x100000, 65537, 10, None) == E
    assert L.hc_cu_census(0x100000, 8, 100001, None) == E


def test_step_counts(hc):
    for R in (2, 3, 8):
        assert hc.hc_step_count(hc.HC_OP_ALLREDUCE, R) == 2 * (R - 1)
        assert hc.hc_step_count(hc.HC_OP_REDUCE_SCATTER, R) == R - 1
        assert hc.hc_step_count(hc.HC_OP_ALL_GATHER, R) == R - 1
        assert hc.hc_step_count(hc.HC_OP_COMPRESSED_ALLREDUCE, R) == 2 * R - 1
        assert hc.hc_step_count(hc.HC_OP_ALLREDUCE_F32_CARRY, R) == 2 * (R - 1)
    assert hc.hc_step_count(hc.HC_OP_COMPRESS_SCOPED, 2) == -1
    assert hc.hc_step_count(hc.HC_OP_ALLREDUCE, 1) == 1
    assert hc.hc_step_count(hc.HC_OP_ALLREDUCE, 0) == -1


def test_status_strings(hc):
    L = _raw(hc)
    for code, text in ((0, b"success"), (1, b"invalid argument"), (3, b"insufficient capacity"),
                       (4, b"corrupt stream"), (5, b"device error")):
        assert L.hc_status_string(code) == text
    assert hc.hc_version().startswith("hc ")


@pytest.mark.parametrize("name,value", [("HC_CHUNK_FRACTION", "0"), ("HC_CHUNK_FRACTION", "1.5"),
                                        ("HC_CHUNK_FRACTION", "0.01x"), ("HC_CU_BUDGET", "-1"),
                                        ("HC_CU_BUDGET", "4097"), ("HC_CU_BUDGET", "8.5")])
def test_malformed_environment_defaults_are_rejected(hc, monkeypatch, name, value):
    """HC_CHUNK_FRACTION and HC_CU_BUDGET replace the defaults of calls that
    pass no options; a malformed value fails every ring call up front,
    naming the variable, before anything is enqueued."""
    L = _raw(hc)
    PP = ctypes.POINTER(ctypes.c_void_p)
    a = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    b = (ctypes.c_void_p * 2)(0x300000, 0x400000)
    monkeypatch.setenv(name, value)
    st = L.hc_allreduce(ctypes.cast(a, PP), ctypes.cast(b, PP), 16, hc.HC_F32, 2, None, None)
    assert st == hc.HC_ERR_INVALID_ARGUMENT
    assert name.encode() in L.hc_last_error()
    st = L.hc_reduce_scatter(ctypes.cast(a, PP), ctypes.cast(b, PP), 8, hc.HC_F32, 2, None, 0, None, None)
    assert st == hc.HC_ERR_INVALID_ARGUMENT and name.encode() in L.hc_last_error()


def test_wellformed_environment_defaults_pass_the_checks(hc, monkeypatch):
    """Valid values pass the up-front checks: the call then fails on the
    next check (here a NULL workspace), not on the environment."""
    L = _raw(hc)
    PP = ctypes.POINTER(ctypes.c_void_p)
    a = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    b = (ctypes.c_void_p * 2)(0x300000, 0x400000)
    monkeypatch.setenv("HC_CHUNK_FRACTION", "0.05")
    monkeypatch.setenv("HC_CU_BUDGET", "8")
    st = L.hc_reduce_scatter(ctypes.cast(a, PP), ctypes.cast(b, PP), 8, hc.HC_F32, 2, None, 0, None, None)
    assert st == hc.HC_ERR_INVALID_ARGUMENT
    assert b"d_ws" in L.hc_last_error()
