"""Pins of the oracle's ring reduce-scatter / all-gather / allreduce.

The ring follows "ResCCL: Resource-Efficient Scheduling for Collective
Communication" section 1 (recvReduceCopy hops, chunk about 1% of the data) and
the AllReduce = ReduceScatter then AllGather split of "Breaking the computation
and communication abstraction barrier in distributed machine learning
workloads" ("The idea").  Pins: brute-force integer sums, hand-derived
order-revealing inputs (tests/golden/ring_order.txt), closed form against the
step simulator, the layout invariants (every rank identical, RS slice r == AR
slice r, AG o RS == AR) and the recursive-summation error bound."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def to_bf16(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_ranks(R, n, dtype, seed, scale=1.0):
    g = np.random.default_rng(seed)
    xs = [(g.standard_normal(n) * scale).astype(np.float32) for _ in range(R)]
    return xs if dtype == "f32" else [to_bf16(x) for x in xs]


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n", [1, 7, 64, 1000, 4099])
def test_integer_inputs_equal_int64_sum(dtype, R, n):
    """|x| <= 16 and R <= 8: every partial is an integer of magnitude <= 128,
    exact in fp32 and bf16, so any order must equal the int64 sum."""
    g = np.random.default_rng(1000 * R + n)
    ints = [g.integers(-16, 17, n) for _ in range(R)]
    xs = [i.astype(np.float32) for i in ints]
    if dtype == "bf16":
        xs = [to_bf16(x) for x in xs]
    expect = np.sum(np.stack(ints), axis=0)
    for out in oracle.allreduce_fold(xs) + oracle.allreduce_ring(xs, chunk=7):
        got = out.astype(np.float64) if dtype == "f32" else bf16_to_f64(out)
        np.testing.assert_array_equal(got, expect.astype(np.float64))


def test_r1_is_identity_and_r2_is_one_ieee_add():
    x = rand_ranks(1, 999, "f32", 3)
    np.testing.assert_array_equal(oracle.allreduce_fold(x)[0], x[0])
    np.testing.assert_array_equal(oracle.allreduce_ring(x)[0], x[0])
    x2 = rand_ranks(2, 1001, "f32", 4)
    # numpy's float32 add is an IEEE binary32 add; with two operands the order is moot
    expect = (x2[0] + x2[1]).view(np.uint32)
    for out in oracle.allreduce_fold(x2):
        np.testing.assert_array_equal(out.view(np.uint32), expect)


# ---------------------------------------------------------------- fold order

def read_order_cases():
    rows = []
    with open(os.path.join(GOLDEN, "ring_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            dtype, R = parts[0], int(parts[1])
            vals = [float(v) for v in parts[2:2 + R]]
            rows.append((dtype, R, vals, float(parts[2 + R])))
    return rows


@pytest.mark.parametrize("case", read_order_cases(), ids=lambda c: f"{c[0]}-R{c[1]}")
def test_fold_order_from_golden(case):
    dtype, R, vals, expect = case
    L = 5
    n = R * L
    xs = [np.zeros(n, dtype=np.float32) for _ in range(R)]
    for j in range(R):
        for k in range(1, R + 1):
            xs[(j + k) % R][j * L:(j + 1) * L] = vals[k - 1]
    if dtype == "bf16":
        xs = [to_bf16(x) for x in xs]
    for outs in (oracle.allreduce_fold(xs), oracle.allreduce_ring(xs, chunk=2)):
        for out in outs:
            got = out.astype(np.float64) if dtype == "f32" else bf16_to_f64(out)
            np.testing.assert_array_equal(got, np.full(n, expect))
    if n % R == 0:
        rs = oracle.reduce_scatter_ring(xs, chunk=3)
        for r in range(R):
            got = rs[r].astype(np.float64) if dtype == "f32" else bf16_to_f64(rs[r])
            np.testing.assert_array_equal(got, np.full(L, expect))


# ---------------------------------------------------------------- two forms agree

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 6, 7, 8])
def test_closed_form_equals_step_simulator(dtype, R):
    for n in (1, 7, R * 33, 1031):
        xs = rand_ranks(R, n, dtype, 17 * R + n)
        fold = oracle.allreduce_fold(xs)
        L = oracle.slice_len(n, R)
        for chunk in sorted({1, 7, 64, oracle.chunk_elems(n), max(L, 1)}):
            ring = oracle.allreduce_ring(xs, chunk=chunk)
            for r in range(R):
                np.testing.assert_array_equal(ring[r], fold[r], err_msg=f"n={n} chunk={chunk} rank={r}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 8])
def test_layout_invariants(dtype, R):
    L = 257
    n = R * L
    xs = rand_ranks(R, n, dtype, 99 + R)
    ar = oracle.allreduce_ring(xs, chunk=50)
    for r in range(1, R):
        np.testing.assert_array_equal(ar[r], ar[0])          # replicated
    rs = oracle.reduce_scatter_ring(xs, chunk=50)
    for r in range(R):
        np.testing.assert_array_equal(rs[r], ar[0][r * L:(r + 1) * L])   # sliced
    ag = oracle.all_gather_ring(rs, chunk=33)
    for r in range(R):
        np.testing.assert_array_equal(ag[r], ar[0])          # AG o RS == AR


def test_all_gather_is_concatenation():
    R, L = 5, 77
    xs = [np.arange(L, dtype=np.float32) + 1000 * r for r in range(R)]
    for out in oracle.all_gather_ring(xs, chunk=10):
        np.testing.assert_array_equal(out, np.concatenate(xs))


# ---------------------------------------------------------------- error bound

def gamma(k, u):
    return k * u / (1 - k * u)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_recursive_summation_bound_fp32(R):
    xs = rand_ranks(R, 20000, "f32", 5 + R)
    out = oracle.allreduce_fold(xs)[0].astype(np.float64)
    X = np.stack([x.astype(np.float64) for x in xs])
    exact = X.sum(axis=0)
    bound = gamma(R - 1, 2.0 ** -24) * np.abs(X).sum(axis=0)
    assert np.all(np.abs(out - exact) <= bound)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_recursive_summation_bound_bf16(R):
    xs = rand_ranks(R, 20000, "bf16", 50 + R, scale=1e-3)
    out = bf16_to_f64(oracle.allreduce_fold(xs)[0])
    X = np.stack([bf16_to_f64(x) for x in xs])
    exact = X.sum(axis=0)
    u = (1 + 2.0 ** -24) * (1 + 2.0 ** -8) - 1     # fp32 add then bf16 rounding per hop
    bound = gamma(R - 1, u) * np.abs(X).sum(axis=0)
    assert np.all(np.abs(out - exact) <= bound)
    # and the bound is not vacuous: most results are inexact (bf16 partials round)
    assert np.mean(out != exact) > 0.3


# ---------------------------------------------------------------- schedule

@pytest.mark.parametrize("R,n,chunk", [(4, 1 << 20, 11264), (8, 1000, 7), (3, 10, 1), (5, 23, 4)])
def test_task_list_shape(R, n, chunk):
    t = oracle.ring_tasks(R, n, chunk)
    L = oracle.slice_len(n, R)
    assert set(np.unique(t["op"])) <= {oracle.OP_RRC, oracle.OP_COPY}
    assert np.all(t["src"] == (t["dst"] - 1) % R)                # ring neighbour
    for op, phase_off in ((oracle.OP_RRC, 2), (oracle.OP_COPY, 1)):
        sub = t[t["op"] == op]
        assert np.all(sub["slice"] == (sub["dst"] - phase_off - sub["step"]) % R)
        for s in range(R - 1):
            for q in range(R):
                tq = sub[(sub["step"] == s) & (sub["dst"] == q)]
                j = (q - phase_off - s) % R
                lo, hi = min(j * L, n), min((j + 1) * L, n)
                covered = np.zeros(n, dtype=np.int32)
                for rec in tq:
                    assert rec["len"] <= chunk
                    covered[rec["off"]:rec["off"] + rec["len"]] += 1
                assert np.all(covered[lo:hi] == 1) and covered.sum() == hi - lo
    # after the reduce-scatter, rank r owns slice r: the last RS step hands q slice q
    last = t[(t["op"] == oracle.OP_RRC) & (t["step"] == R - 2)]
    assert np.all(last["slice"] == last["dst"])


def test_chunk_is_about_one_percent():
    for n, align in ((1 << 20, 1024), (1 << 26, 1024), (1 << 25, 16384), (1 << 28, 1024), (5, 1024)):
        c = oracle.chunk_elems(n, align)
        assert c % align == 0
        assert c >= n / 100 and c < n / 100 + align


# ------------------------------------------------ the fold at chosen indices

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("R", [1, 2, 3, 5, 7, 8, 16, 33, 64])
def test_fold_at_equals_whole_fold_at_every_index(dtype, R):
    """or_allreduce_fold_at is the checker of the full-size GPU tests, which
    compare outputs too large for the whole fold at once.  At every index of
    buffers where R divides n and where it does not (short and empty last
    slices), it must return exactly the whole fold's word, in any index order
    and with repeats."""
    for n in (R * 37, R * 37 + 1, R * 37 + R - 1, 1, 5):
        xs = rand_ranks(R, n, dtype, 7000 + 97 * R + n)
        whole = oracle.allreduce_fold(xs)[0]
        idx = np.arange(n, dtype=np.uint64)
        np.testing.assert_array_equal(oracle.allreduce_fold_at(xs, idx), whole)
        perm = np.random.default_rng(n).permutation(n).astype(np.uint64)
        rep = np.concatenate([perm, perm[: max(1, n // 3)]])
        np.testing.assert_array_equal(oracle.allreduce_fold_at(xs, rep), whole[rep.astype(np.int64)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fold_at_slice_edges_order_revealing(dtype):
    """Every slice's first and last index and the tail, with inputs whose sum
    depends on the fold order (x[j+1] = 1, x[j+2] = 2^24, x[j+3] = -2^24 in
    fp32; 1, 2^8, -2^8 in bf16): a fold started at the wrong rank or a slice
    index off by one gives another word there."""
    R, L = 4, 9
    n = R * L - 2          # the last slice is short
    big = 2.0 ** 24 if dtype == "f32" else 2.0 ** 8
    vals = np.zeros((R, n), dtype=np.float64)
    for i in range(n):
        j = i // L
        vals[(j + 1) % R, i] = 1.0
        vals[(j + 2) % R, i] = big
        vals[(j + 3) % R, i] = -big
    xs = [v.astype(np.float32) for v in vals]
    if dtype == "bf16":
        xs = [to_bf16(x) for x in xs]
    edges = sorted({0, n - 1, *[j * L for j in range(R) if j * L < n],
                    *[min(n, (j + 1) * L) - 1 for j in range(R)]})
    got = oracle.allreduce_fold_at(xs, np.array(edges, dtype=np.uint64))
    got = got.astype(np.float64) if dtype == "f32" else bf16_to_f64(got)
    # ((1 + big) - big) + 0: the 1 is lost to rounding in the first hop
    np.testing.assert_array_equal(got, np.zeros(len(edges)))
    np.testing.assert_array_equal(oracle.allreduce_fold_at(xs, np.array(edges, dtype=np.uint64)),
                                  oracle.allreduce_fold(xs)[0][edges])


def test_fold_at_rejects_out_of_range_index():
    xs = rand_ranks(3, 10, "f32", 5)
    with pytest.raises(ValueError):
        oracle.allreduce_fold_at(xs, np.array([10], dtype=np.uint64))
