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
        assert rec["bytes_per_launch"] >= rec["alg_bytes_per_launch"] * 0.99, key
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
