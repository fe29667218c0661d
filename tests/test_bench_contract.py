"""bench.py's command-line contract that holds without a GPU: runs across
several GPUs are refused with a message and a non-zero exit, the traffic
records are taken only on the kernel source they were measured on, and the
roofline object carries the fields the bench line promises."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        msg = json.loads(r.stdout.strip().splitlines()[-1])
        assert "one GPU" in msg["error"] and msg["n_gpus"] == int(n)


def test_traffic_record_needs_the_measured_source():
    # every recorded kernel names a source hash; a record is used only while
    # the sources hash to it
    data = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))
    assert data
    for key, rec in data.items():
        assert len(rec["source_hash"]) == 16, key
        # a kernel that re-reads what it wrote within the launch can be served
        # from cache: it then states its compulsory bytes (inputs read once,
        # outputs written once), below which no count can fall
        floor = rec.get("compulsory_bytes_per_launch", rec["alg_bytes_per_launch"])
        assert floor <= rec["alg_bytes_per_launch"], key
        assert rec["bytes_per_launch"] >= floor * 0.99, key
    files = ["collective_communication_amd/csrc/ring_kernels.hip", "collective_communication_amd/csrc/common.hpp"]
    rec = data["reduce_step:ring_bf16"]
    expect = rec["bytes_per_launch"] if rec["source_hash"] == bench.kernel_hash(files) else None
    assert bench.load_traffic("reduce_step", "ring_bf16", files) == expect
    assert bench.load_traffic("no_such_kernel", "ring_bf16", files) is None


def test_roofline_object_fields():
    r = bench.roofline_obj("k", 8_000_000_000, 1.0, 123, "d")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 8000.0) < 1e-6 and abs(r["frac"] - 1.0) < 1e-9
    assert r["traffic"] == 123 and r["alg_bytes_per_launch"] == 8_000_000_000
    assert "traffic_source" in r and "recorded" in r["traffic_source"]
    assert "traffic_source" not in bench.roofline_obj("k", 1, 1.0, None)


def test_contention_rate_matches_the_oracle():
    """The contention-rate arithmetic the bench line reports equals the
    oracle's on hand-built interval sets (known integrals) and on random
    ones: GEMM calls back to back, one or several communication intervals."""
    import numpy as np
    import oracle

    cases = [
        ([(0, 10)], [(2, 7, 32)], 256, 0.0625),            # 5/10 of the time at 32/256
        ([(0, 4), (4, 8)], [(0, 8, 8)], 256, 8 / 256),     # communication spans every GEMM
        ([(0, 10)], [(20, 30, 64)], 256, 0.0),             # no overlap
        ([(0, 2), (5, 7)], [(1, 6, 128)], 256, 0.25),      # 2 of 4 compute units of time at 1/2
    ]
    for comp, comm, ncu, want in cases:
        assert abs(bench.contention_rate(comp, comm, ncu) - want) < 1e-12
        assert abs(oracle.contention_rate(comp, comm, ncu) - want) < 1e-12
    g = np.random.default_rng(11)
    for _ in range(200):
        edges = np.cumsum(g.uniform(0.1, 2.0, g.integers(1, 12)))
        comp = [(float(a), float(b)) for a, b in zip(np.r_[0.0, edges[:-1]], edges)]
        comm = []
        for _ in range(g.integers(1, 4)):
            t0 = float(g.uniform(-2, edges[-1] + 1))
            comm.append((t0, t0 + float(g.uniform(0.0, 6.0)), int(g.integers(1, 257))))
        a = bench.contention_rate(comp, comm, 256)
        b = oracle.contention_rate(comp, comm, 256)
        assert abs(a - b) < 1e-12, (comp, comm, a, b)
    assert bench.contention_rate([], [(0, 1, 8)], 256) is None


def test_cpu_baseline_names_its_host():
    info = bench.host_info()
    assert info["nproc"] >= 1 and isinstance(info["cpu_model"], str)
    rec = bench.oracle_timed(lambda: sum(range(1000)), 1000, "a sample")
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["nproc"] == info["nproc"]
    assert "cpu_model" in rec


def test_ring_metric_names_its_rank_count():
    # the headline line carries the metric string as given; another rank count names its own
    assert bench.ring_metric(8) == bench.METRIC
    assert "R=4," in bench.ring_metric(4) and "R=8" not in bench.ring_metric(4)
