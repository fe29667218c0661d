#!/usr/bin/env python3
"""Benchmark of the emulated ring AllReduce data path on one MI355X.

Default workload (the one the printed JSON line is about): ring AllReduce
(sum) over R=8 emulated ranks of 2^26 bf16 elements each, N(0, 1e-3) with 1%
exact zeros, fp32 accumulation per hop with bf16 nearest-even output, chunk
~1% of the buffer, reduce-scatter then all-gather.  One "step" is one whole
allreduce (14 ring steps) over inputs already resident in HBM.

Other workloads (--workload): ring_f32 (R=4 x 2^20 fp32), ring_bf16_carry
(the default ring with fp32 partials and one final rounding), codec (2^28 bf16
compress/decompress of weights, activations, gradients), compressed (the
fused compressed ring, R=8 x 2^25 bf16), contention (R=8 reduce-scatter of
2^28 bf16 on a CU-budget stream next to a bf16 8192^3 GEMM, plus the matching
all-gather on CU copy kernels and on the DMA engines), fused_sgd (the allreduce
of R=8 x 2^26 bf16 gradients fused with an SGD update of the weights),
table_scope (the codec's code tables per block, per group of blocks or global,
and the per-block encoder in three global rounds, on 2^28 bf16 weights,
gradients and a multi-layer gradient bucket), entropy
(the HCE1 variant with per-block Huffman codes for the exponent, next to the
fixed-length codec on the same 2^28 tensors), hop_sizes (the reduce-scatter
hop at 2^24..2^28 elements per rank under each store policy, with and without
a cold Infinity Cache), rs_budget (the contention test's reduce-scatter on
k = 8, 16, 32 CUs and on all CUs, without the GEMM), compressed_schedules (the
compressed ring at R = 2, 4, 8 and 2^18..2^25 elements per rank, one launch per
ring step against one launch for the whole allreduce).  Each prints one JSON
line of its own.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
The headline time is K back-to-back calls with nothing else on the stream.
The per-kernel figures come from a second pass of K calls in which every
ring step's kernels stamp two HIP events with their own start and end times
(hc_opts_t.step_events in kernel-stamp mode, hipExtLaunchKernel): the same
durations a kernel trace reports.  That pass launches through the event
path, so it is kept out of the headline time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 MFMA, published
N_CU = 256

METRIC = "AllReduce algbw GB/s and achieved HBM GB/s (% of peak), R=8, 1 MI355X"


def ring_metric(R: int) -> str:
    """The headline metric (R=8), with the rank count of a workload that uses another."""
    return METRIC.replace("R=8,", f"R={R},")
# sources whose change voids the recorded traffic counters of a kernel
CODEC_FILES = ["collective_communication_amd/csrc/codec_kernels.hip", "collective_communication_amd/csrc/codec.hpp",
               "collective_communication_amd/csrc/lookback.hpp", "collective_communication_amd/csrc/common.hpp",
               "collective_communication_amd/csrc/car.hpp", "collective_communication_amd/csrc/car_chain.hip"]
ENTROPY_FILES = ["collective_communication_amd/csrc/entropy_kernels.hip", "collective_communication_amd/csrc/codec.hpp",
                 "collective_communication_amd/csrc/lookback.hpp", "collective_communication_amd/csrc/common.hpp"]
RING_FILES = ["collective_communication_amd/csrc/ring_kernels.hip", "collective_communication_amd/csrc/common.hpp"]


def kernel_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, files):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(f"{kernel}:{workload}")
    if not rec or rec.get("source_hash") != kernel_hash(files):
        return None
    return rec.get("bytes_per_launch")


def timed_ms(call, steps: int) -> float:
    """Average ms of `call` over `steps` back-to-back calls on the current
    stream, bracketed by device synchronisation and two events."""
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def hbm_ceiling(operand_bytes: int) -> dict:
    """Runs the hbm_ceiling tool built in measure/ (streaming add, copy and
    read kernels at the given operand size) and returns its JSON object, or
    {"error": ...}."""
    tool = os.path.join(ROOT, "measure", "hbm_ceiling")
    try:
        r = subprocess.run([tool, str(operand_bytes >> 20)], capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            return {"error": r.stderr[-2000:]}
        return json.loads(r.stdout.strip().splitlines()[-1])
    except (OSError, ValueError, subprocess.TimeoutExpired) as exc:
        return {"error": repr(exc)}


def roofline_obj(kernel: str, alg_bytes: int, ms: float, traffic=None, duration: str | None = None):
    """The dominant kernel against MI355X's HBM peak: algorithmic bytes per
    launch over the launch's duration (HIP events on its stream, stamped by
    the kernel's own start and end where a step-event pass measures it)."""
    gbps = alg_bytes / (ms / 1e3) / 1e9
    d = {"bound": "hbm", "kernel": kernel, "achieved": round(gbps, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": traffic, "alg_bytes_per_launch": int(alg_bytes),
         "launch_ms": round(ms, 6)}
    if duration:
        d["duration"] = duration
    if traffic is not None:
        d["traffic_source"] = TRAFFIC_SOURCE
    return d


def host_info() -> dict:
    """The host the oracle runs on: logical CPUs this process may use and the
    CPU model."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count() or 0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": nproc, "cpu_model": model}


def contention_rate(compute, comm, n_cu: float):
    """The contention rate of "HOCCL: Offloading Collective Communication from
    GPU Cores to Accelerate Distributed Training" (section 2: the share of
    compute units that communication holds while compute kernels run), read
    as I = integral of C(t) * CU(t) / n_cu over integral of C(t), with C(t) = 1
    while any compute interval (t0, t1) runs and CU(t) the compute units of
    the communication intervals (t0, t1, cus) running at t.  Returns None when
    no compute ran."""
    pts = sorted({t for a, b in compute for t in (a, b)} | {t for a, b, _ in comm for t in (a, b)})
    num = den = 0.0
    for a, b in zip(pts, pts[1:]):
        mid = 0.5 * (a + b)
        if not any(c0 <= mid < c1 for c0, c1 in compute):
            continue
        cu = sum(k for m0, m1, k in comm if m0 <= mid < m1)
        den += b - a
        num += (b - a) * cu / n_cu
    return num / den if den > 0 else None


def oracle_timed(fn, nbytes: int, sample: str, unit: str = "GB/s"):
    """The oracle as it stands, one host thread, on a bounded sample; nbytes
    is what the sample moves in the metric's sense."""
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{sample}; {dt:.2f} s", **host_info()}


TRAFFIC_SOURCE = ("recorded, not measured in this run: rocprofv3 FETCH_SIZE and WRITE_SIZE per launch from "
                  "profiles/pmc_traffic.json, taken on the same kernel source (matched by source hash), "
                  "FETCH_SIZE scaled by the plain-copy calibration factor")


def cpu_baseline_ring(R: int, n_sample: int):
    """The oracle's ring step simulator, as it stands, on a bounded sample of
    the same workload (first n_sample elements of every rank), one thread."""
    import oracle
    from collective_communication_amd import inputs

    xs = [inputs.host_bits(t) for t in inputs.ring_inputs_cuda("ring_bf16", R, n_sample)]
    t0 = time.perf_counter()
    oracle.allreduce_ring(xs)
    dt = time.perf_counter() - t0
    return {"value": round(n_sample * 2 / dt / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"R={R} ranks x {n_sample} bf16 elements (same recipe), ring step simulator, "
                      f"{dt:.2f} s", **host_info()}


def bench_ring(args, workload: str):
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    if workload == "ring_bf16":
        R, n, es, dtype = 8, 1 << 26, 2, "bf16"
    else:
        R, n, es, dtype = 4, 1 << 20, 4, "f32"
    send = inputs.ring_inputs_cuda(workload, R, n)
    recv = [torch.empty_like(s) for s in send]
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE, R)
    for _ in range(args.warmup):
        hc.hc_allreduce(send, recv)
    ms = timed_ms(lambda: hc.hc_allreduce(send, recv), args.steps)
    # Per-kernel durations: the same calls again, every step's kernels
    # stamping their own start and end (kept out of the headline time).
    evsets = [hc.StepEvents.for_steps(steps, mode=1) for _ in range(args.steps)]
    for k in range(args.steps):
        hc.hc_allreduce(send, recv, step_events=evsets[k])
    torch.cuda.synchronize()
    # Step intervals: R-2 plain reduce-scatter steps, the last one (a
    # reduce-and-send that also writes each slice into the next rank's
    # output), the first all-gather step (empty: done by the step before) and
    # R-2 copy steps.
    red, fused, cpy = [], [], []
    for ev in evsets:
        d = ev.elapsed_ms()
        red += d[: R - 2]
        fused.append(d[R - 2])
        cpy += d[R:]
    avg_red, avg_cpy = sum(red) / len(red), sum(cpy) / len(cpy)
    avg_fused = sum(fused) / len(fused)
    L = n // R
    rs_bytes = 3 * es * n * (R - 2) + 4 * es * n       # per allreduce; the last step writes twice
    ag_bytes = 2 * es * n * (R - 2)
    alg_bytes = rs_bytes + ag_bytes
    method_bytes = (3 + 2) * es * n * (R - 1)            # R-1 reduce hops and R-1 copy hops
    red_launch_bytes = 3 * es * n                        # one reduce step: R receivers x L elements
    algbw = n * es / (ms / 1e3) / 1e9
    hbm = alg_bytes / (ms / 1e3) / 1e9
    achieved = red_launch_bytes / (avg_red / 1e3) / 1e9
    traffic = load_traffic("reduce_step", workload, RING_FILES)
    # Allreduces whose R buffers hold at most HC_CHAIN_MAX_BYTES (256 MiB by
    # default, as in the library) run as one launch that carries each tile
    # through every hop; the per-step stamps above come from the
    # step-per-launch schedule, which step events always select.
    chain_max = int(os.environ.get("HC_CHAIN_MAX_BYTES", str(256 << 20)) or 0)
    one_launch = R * n * es <= chain_max
    line = {
        "metric": ring_metric(R), "value": round(algbw, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"emulated ring allreduce (sum), R={R} ranks x {n} {dtype} per rank, "
                               f"{'N(0,1e-3) with 1% zeros, fp32 add + bf16 RNE per hop' if dtype == 'bf16' else 'N(0,1), fp32 add per hop'}, "
                               f"chunk ~1%, reduce-scatter then all-gather",
                   "ranks": R, "elems_per_rank": n, "slice": L, "chunk": hc.hc_chunk_elems(n)},
        "busbw_gbps": round(algbw * 2 * (R - 1) / R, 3),
        "hbm_gbps": round(hbm, 2), "hbm_frac_of_peak": round(hbm / PEAK_HBM_GBPS, 4),
        "alg_bytes_per_step": alg_bytes,
        "alg_bytes_basis": "what this implementation moves: R-2 reduce hops (2 reads, 1 write), one "
                           "reduce-and-send hop (2 reads, 2 writes) that also does the first all-gather copy, "
                           "R-2 copy hops",
        "method_alg_bytes_per_step": method_bytes,
        "method_hbm_gbps": round(method_bytes / (ms / 1e3) / 1e9, 2),
        "method_hbm_frac_of_peak": round(method_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
        "method_bytes_basis": "the ring method's own accesses: R-1 reduce hops (2 reads, 1 write) and R-1 copy "
                              "hops (1 read, 1 write)",
        "reduce_launch_ms": round(avg_red, 6), "reduce_send_launch_ms": round(avg_fused, 6),
        "copy_launch_ms": round(avg_cpy, 6),
        "copy_launch_gbps": round(2 * es * n / (avg_cpy / 1e3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "step_kernel<reduce> (one reduce-scatter step)",
                     "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": red_launch_bytes, "launch_ms": round(avg_red, 6),
                     "duration": "mean reduce-scatter step by its kernel's start and end stamps (HIP events)"},
        "schedule": "one launch, each tile through every hop" if one_launch else "one launch per ring step",
    }
    if one_launch:
        # the headline call is a single chain_kernel launch: its bytes are the
        # whole allreduce's, its duration the call's (back to back, launch gaps
        # included); the step-per-launch figures stay beside it
        line["step_schedule"] = {"reduce_launch_ms": line.pop("reduce_launch_ms"),
                                 "reduce_send_launch_ms": line.pop("reduce_send_launch_ms"),
                                 "copy_launch_ms": line.pop("copy_launch_ms"),
                                 "copy_launch_gbps": line.pop("copy_launch_gbps"),
                                 "roofline": line["roofline"]}
        line["roofline"] = {"bound": "hbm", "kernel": "chain_kernel (the whole allreduce in one launch)",
                            "achieved": round(hbm, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(hbm / PEAK_HBM_GBPS, 4),
                            "traffic": load_traffic("chain", workload, RING_FILES),
                            "alg_bytes_per_launch": alg_bytes, "launch_ms": round(ms, 6),
                            "duration": "per call, back to back (HIP events around the calls)"}
    if line["roofline"]["traffic"] is not None:
        line["roofline"]["traffic_source"] = TRAFFIC_SOURCE
    if workload == "ring_bf16":
        # What a plain streaming kernel with the reduce hop's traffic (two
        # reads, one write of 128 MiB operands, the same tiling) reaches on
        # this GPU, measured in a process of its own: the practical ceiling
        # the hop is held against next to the published peak.
        ceil = hbm_ceiling(n * es)
        line["hbm_ceiling"] = ceil
        if "add" in ceil:
            line["roofline"]["practical_ceiling_gbps"] = ceil["add"]["gbps"]
            line["roofline"]["frac_of_practical_ceiling"] = round(achieved / ceil["add"]["gbps"], 4)
    if not args.no_cpu_baseline and workload == "ring_bf16":
        line["cpu_baseline"] = cpu_baseline_ring(R, args.cpu_sample)
    elif not args.no_cpu_baseline:
        import oracle

        xs = [inputs.host_bits(t) for t in send]
        line["cpu_baseline"] = oracle_timed(lambda: oracle.allreduce_ring(xs), n * es,
                                            f"the whole workload (R={R} x {n} {dtype}), ring step simulator")
    return line


def bench_ring_carry(args):
    """The bf16 ring with fp32 partials and one final rounding
    (hc_allreduce_bf16_f32carry) on the default workload, with the per-hop
    ring timed beside it, and the error of both against the exact sum on a
    sample of elements."""
    import numpy as np
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, n = 8, 1 << 26
    send = inputs.ring_inputs_cuda("ring_bf16", R, n)
    recv = [torch.empty_like(s) for s in send]
    hop = [torch.empty_like(s) for s in send]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_ALLREDUCE_F32_CARRY, n, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        hc.hc_allreduce_bf16_f32carry(send, recv, n, ws)
        hc.hc_allreduce(send, hop)
    ms = timed_ms(lambda: hc.hc_allreduce_bf16_f32carry(send, recv, n, ws), args.steps)
    ms_hop = timed_ms(lambda: hc.hc_allreduce(send, hop), args.steps)
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE_F32_CARRY, R)
    evsets = [hc.StepEvents.for_steps(steps, mode=1) for _ in range(args.steps)]
    for k in range(args.steps):
        hc.hc_allreduce_bf16_f32carry(send, recv, n, ws, step_events=evsets[k])
    torch.cuda.synchronize()
    first, mid, last, cpy = [], [], [], []
    for ev in evsets:
        d = ev.elapsed_ms()
        first.append(d[0])
        mid += d[1:R - 2]
        last.append(d[R - 2])
        cpy += d[R:]   # d[R - 1], the first all-gather step, is empty: the last hop sent it
    avg = lambda v: sum(v) / len(v)
    # bytes per element of one step (N elements per step over the R receivers):
    # first hop 2 + 2 read, 4 written; a middle hop 4 + 2 read, 4 written; the
    # last hop 4 + 2 read, 2 + 2 written (the rounded sum into its owner and
    # into the next rank); R-2 all-gather copies 2 read, 2 written.
    alg_bytes = n * (8 + 10 * (R - 3) + 10 + 4 * (R - 2))
    mid_bytes = 10 * n
    algbw = n * 2 / (ms / 1e3) / 1e9
    # Error against the exact sum on 65,536 elements (fp64 holds every 8-term
    # bf16 sum exactly here): the share of results that are the exact sum
    # correctly rounded (within half a bf16 ulp of it), and the error in bf16
    # ulps of the sum of magnitudes (the scale the summation error bound uses).
    g = np.random.default_rng(3)
    idx = torch.from_numpy(g.integers(0, n, 1 << 16).astype(np.int64)).to("cuda")
    vals = (np.stack([inputs.host_bits(s[idx]) for s in send]).astype(np.uint32) << 16).view(np.float32)
    exact = vals.astype(np.float64).sum(axis=0)
    mag = np.abs(vals.astype(np.float64)).sum(axis=0)

    def bf16_ulp(x):
        nz = x != 0
        return np.where(nz, np.exp2(np.floor(np.log2(np.where(nz, np.abs(x), 1.0))) - 7), 0.0)

    def ulp_err(t):
        got = (inputs.host_bits(t[idx]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        d = np.abs(got - exact)
        ok = np.where(exact != 0, d <= 0.5 * bf16_ulp(exact), got == 0)
        scale = np.where(mag != 0, bf16_ulp(mag), 1.0)
        e = d / scale
        return {"correctly_rounded": round(float(ok.mean()), 5),
                "max_ulps_of_sum_of_magnitudes": round(float(e.max()), 4),
                "mean_ulps_of_sum_of_magnitudes": round(float(e.mean()), 5)}

    line = {
        "metric": METRIC, "value": round(algbw, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"emulated ring allreduce (sum) with fp32 partials and one final bf16 rounding, "
                               f"R={R} ranks x {n} bf16 per rank, N(0,1e-3) with 1% zeros, chunk ~1%, "
                               f"reduce-scatter then all-gather",
                   "ranks": R, "elems_per_rank": n, "chunk": hc.hc_chunk_elems(n)},
        "hbm_gbps": round(alg_bytes / (ms / 1e3) / 1e9, 2),
        "hbm_frac_of_peak": round(alg_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
        "alg_bytes_per_step": alg_bytes,
        "per_hop_ms_per_step": round(ms_hop, 6),
        "per_hop_algbw_gbps": round(n * 2 / (ms_hop / 1e3) / 1e9, 3),
        "first_rs_ms": round(avg(first), 6), "middle_rs_ms": round(avg(mid), 6), "last_rs_ms": round(avg(last), 6),
        "copy_ms": round(avg(cpy), 6),
        "error_vs_exact": {"f32_carry": ulp_err(recv[0]), "per_hop": ulp_err(hop[0])},
        "roofline": roofline_obj("carry_kernel<fp32 in, fp32 out> (a middle reduce-scatter step)", mid_bytes,
                                 avg(mid), None, "mean middle reduce-scatter step by its kernel's start and "
                                                 "end stamps (HIP events)"),
    }
    if not args.no_cpu_baseline:
        import oracle

        m = min(n, args.cpu_sample)
        xs = [inputs.host_bits(s[:m]) for s in send]
        line["cpu_baseline"] = oracle_timed(lambda: oracle.allreduce_fold_f32carry(xs), m * 2,
                                            f"R={R} x {m} bf16 (the first {m} elements of every rank), "
                                            f"the oracle's fp32-carry fold")
    return line


def bench_codec(args):
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    n = 1 << 28
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS, n, 1), dtype=torch.uint8, device="cuda")
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = {}
    for name, maker in (("weights", lambda: inputs.normal_bf16_cuda("codec", 0, n, 0.02)),
                        ("activations", lambda: inputs.activation_bf16_cuda("codec", 1, n)),
                        ("gradients", lambda: inputs.normal_bf16_cuda("codec", 2, n, 1e-4))):
        x = maker()
        for _ in range(args.warmup):
            hc.hc_compress_bf16(x, n, out, nbytes, ws)
            hc.hc_decompress_bf16(out, cap, back, n, status)
        torch.cuda.synchronize()
        size = int(nbytes.item())
        ok = int(status.item()) == 0 and torch.equal(back.view(torch.int16), x.view(torch.int16))
        # K back-to-back calls of each (the same input gives the same stream).
        mc = timed_ms(lambda: hc.hc_compress_bf16(x, n, out, nbytes, ws), args.steps)
        md = timed_ms(lambda: hc.hc_decompress_bf16(out, cap, back, n, status), args.steps)
        ok = ok and int(nbytes.item()) == size and int(status.item()) == 0 and \
            torch.equal(back.view(torch.int16), x.view(torch.int16))
        raw = 2 * n
        rows[name] = {"ratio": round(size / raw, 5), "compressed_bytes": size,
                      "compress_ms": round(mc, 4), "decompress_ms": round(md, 4),
                      "compress_raw_gbps": round(raw / mc / 1e6, 1), "decompress_raw_gbps": round(raw / md / 1e6, 1),
                      "compress_hbm_gbps": round((raw + size) / mc / 1e6, 1),
                      "decompress_hbm_gbps": round((raw + size) / md / 1e6, 1),
                      "round_trip_exact": ok}
        del x
    worst = min(min(r["compress_hbm_gbps"], r["decompress_hbm_gbps"]) for r in rows.values())
    w = rows["weights"]
    codec_files = CODEC_FILES
    line = {"metric": "HCZ1 bf16 codec throughput (HBM GB/s, raw GB/s) and ratio, 2^28 elements",
            "value": worst, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "standalone lossless bf16 codec, 2^28 elements per tensor"},
            "tensors": rows, "hbm_frac_of_peak_worst": round(worst / PEAK_HBM_GBPS, 4),
            "roofline": roofline_obj("compress_kernel (weights)", 2 * n + w["compressed_bytes"], w["compress_ms"],
                                     load_traffic("compress", "codec", codec_files),
                                     "per hc_compress_bf16 call, back to back: the kernel and the clear of its look-back "
                                     "workspace"),
            "roofline_decompress": roofline_obj("decompress_kernel (weights)", 2 * n + w["compressed_bytes"],
                                                w["decompress_ms"], load_traffic("decompress", "codec", codec_files),
                                                "per hc_decompress_bf16 call, back to back: the kernel, the status clear and the "
                                                "corrupt-stream check")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 26
        host = inputs.host_bits(inputs.normal_bf16_cuda("codec", 0, n, 0.02)[:m])
        stream = oracle.compress(host)
        line["cpu_baseline"] = oracle_timed(lambda: oracle.compress(host), 2 * m + len(stream),
                                            f"oracle compress of the first {m} elements of the weights tensor "
                                            "(HBM-equivalent bytes: input + stream)")
    return line


def bench_entropy(args):
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    n = 1 << 28
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_ENTROPY, n, 1), dtype=torch.uint8, device="cuda")
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    coders = {"fixed": (hc.hc_compress_bf16, hc.hc_decompress_bf16),
              "entropy": (hc.hc_compress_bf16_entropy, hc.hc_decompress_bf16_entropy)}
    rows = {}
    for name, maker in (("weights", lambda: inputs.normal_bf16_cuda("codec", 0, n, 0.02)),
                        ("activations", lambda: inputs.activation_bf16_cuda("codec", 1, n)),
                        ("gradients", lambda: inputs.normal_bf16_cuda("codec", 2, n, 1e-4)),
                        ("bucket", lambda: inputs.bucket_bf16_cuda("bucket", 0, n))):
        x = maker()
        row = {}
        for label, (comp, decomp) in coders.items():
            for _ in range(args.warmup):
                comp(x, n, out, nbytes, ws)
            mc = timed_ms(lambda: comp(x, n, out, nbytes, ws), args.steps)
            size = int(nbytes.item())
            md = timed_ms(lambda: decomp(out, cap, back, n, status), args.steps)
            ok = int(status.item()) == 0 and torch.equal(back.view(torch.int16), x.view(torch.int16))
            raw = 2 * n
            row[label] = {"ratio": round(size / raw, 5), "compressed_bytes": size, "compress_ms": round(mc, 4),
                          "decompress_ms": round(md, 4), "compress_raw_gbps": round(raw / mc / 1e6, 1),
                          "decompress_raw_gbps": round(raw / md / 1e6, 1),
                          "compress_hbm_gbps": round((raw + size) / mc / 1e6, 1),
                          "decompress_hbm_gbps": round((raw + size) / md / 1e6, 1), "round_trip_exact": ok}
        row["entropy_size_saving"] = round(1 - row["entropy"]["ratio"] / row["fixed"]["ratio"], 4)
        rows[name] = row
        del x
    w = rows["weights"]["entropy"]
    line = {"metric": "HCE1 (Huffman exponent) bf16 codec: compressed/raw size and throughput, 2^28 elements",
            "value": min(r["entropy"]["compress_hbm_gbps"] for r in rows.values()), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "dtype": "u8",
            "data": "synthetic",
            "config": {"workload": "entropy-coded exponent variant next to the fixed-length codec, 2^28 bf16 per "
                                   "tensor (weights, activations, gradients, gradient bucket)"},
            "weights_ratio": w["ratio"], "tensors": rows,
            "roofline": roofline_obj("hce_compress_kernel (weights)", 2 * n + w["compressed_bytes"], w["compress_ms"],
                                     load_traffic("hce_compress", "entropy", ENTROPY_FILES),
                                     "per hc_compress_bf16_entropy call: the kernel and the clear of its "
                                     "look-back workspace"),
            "roofline_decompress": roofline_obj("hce_decompress_kernel (weights)", 2 * n + w["compressed_bytes"],
                                                w["decompress_ms"], load_traffic("hce_decompress", "entropy",
                                                                                 ENTROPY_FILES),
                                                "per hc_decompress_bf16_entropy call: the kernel, the status clear "
                                                "and the corrupt-stream check")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 26
        host = inputs.host_bits(inputs.normal_bf16_cuda("codec", 0, n, 0.02)[:m])
        stream = oracle.hce_compress(host)
        line["cpu_baseline"] = oracle_timed(lambda: oracle.hce_compress(host), 2 * m + len(stream),
                                            f"oracle HCE1 compress of the first {m} elements of the weights tensor "
                                            "(HBM-equivalent bytes: input + stream)")
    return line


def bench_table_scope(args):
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    n = 1 << 28
    cap = hc.hc_compress_bound_bf16(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    nbytes = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_SCOPED, n, 1), dtype=torch.uint8, device="cuda")
    back = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    scopes = [("per_block", None), ("per_block_3_rounds", "staged"), ("group_1", 1), ("group_8", 8),
              ("group_64", 64), ("global", 0)]
    ws3 = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESS_STAGED, n, 1), dtype=torch.uint8, device="cuda")
    rows = {}
    for name, maker in (("weights", lambda: inputs.normal_bf16_cuda("codec", 0, n, 0.02)),
                        ("gradients", lambda: inputs.normal_bf16_cuda("codec", 2, n, 1e-4)),
                        ("bucket", lambda: inputs.bucket_bf16_cuda("bucket", 0, n))):
        x = maker()
        row = {}
        for label, group in scopes:
            if group is None:
                call = lambda: hc.hc_compress_bf16(x, n, out, nbytes, ws)
            elif group == "staged":
                call = lambda: hc.hc_compress_bf16_staged(x, n, out, nbytes, ws3)
            else:
                call = lambda g=group: hc.hc_compress_bf16_scoped(x, n, out, nbytes, g, ws)
            for _ in range(args.warmup):
                call()
            ms = timed_ms(call, args.steps)
            size = int(nbytes.item())
            hc.hc_decompress_bf16(out, cap, back, n, status)
            torch.cuda.synchronize()
            ok = int(status.item()) == 0 and torch.equal(back.view(torch.int16), x.view(torch.int16))
            row[label] = {"ratio": round(size / (2 * n), 5), "compressed_bytes": size, "compress_ms": round(ms, 4),
                          "compress_raw_gbps": round(2 * n / ms / 1e6, 1), "round_trip_exact": ok}
        rows[name] = row
        del x
    b = rows["bucket"]
    g = b["global"]
    line = {"metric": "HCZ1 compressed/raw size of a 2^28 bf16 gradient bucket with per-block code tables",
            "value": b["per_block"]["ratio"], "unit": "ratio", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "higher_is_better": False, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "code-table scope sweep: per block, groups of 1/8/64 blocks, one global "
                                   "table; 2^28 bf16 per tensor"},
            "global_over_per_block_size": round(b["global"]["ratio"] / b["per_block"]["ratio"], 4),
            "three_rounds_over_one_round_time": round(b["per_block_3_rounds"]["compress_ms"]
                                                      / b["per_block"]["compress_ms"], 3),
            "tensors": rows,
            "roofline": roofline_obj("hc_compress_bf16_scoped, one global table (bucket)",
                                     2 * n + g["compressed_bytes"], g["compress_ms"], None,
                                     "per call: the histogram pass, the four small scope kernels, the workspace "
                                     "clears and compress_kernel<true>; bytes are the input and the stream only")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 26
        host = inputs.host_bits(inputs.bucket_bf16_cuda("bucket", 0, n)[:m])
        stream = oracle.compress_scoped(host, 0)
        line["cpu_baseline"] = oracle_timed(lambda: oracle.compress_scoped(host, 0), 2 * m + len(stream),
                                            f"oracle compress_scoped (one global table) of the first {m} elements of "
                                            "the bucket (HBM-equivalent bytes: input + stream)")
    return line


def bench_compressed(args):
    """The fused compressed ring allreduce, R=8 x 2^25 bf16.  The library runs
    it as one launch (car_chain_kernel: each codec block of each slice through
    every hop); the headline is K back-to-back calls, and the roofline is that
    launch over the whole call's algorithmic bytes.  Beside it, untimed in the
    headline: the step-per-launch schedule (HC_CHAIN_MAX_BYTES=0) back to
    back, and its per-step kernel stamps (step events select that schedule).
    Both schedules warm up for at least 30 calls: under back-to-back load the
    GPU's clock first drops (to about 1.9 GHz within five calls of this
    workload) and settles near 2.3 GHz after about 25, and the timed region
    should see the settled clock."""
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, n = 8, 1 << 25
    send = inputs.ring_inputs_cuda("compressed", R, n)
    recv = [torch.empty_like(s) for s in send]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), dtype=torch.uint8, device="cuda")
    wire = torch.zeros(1, dtype=torch.int64, device="cuda")
    steps = hc.hc_step_count(hc.HC_OP_COMPRESSED_ALLREDUCE, R)

    def call():
        hc.hc_compressed_allreduce(send, recv, n, ws)

    warmup = max(args.warmup, 30)
    for _ in range(warmup):
        call()
    ms = timed_ms(call, args.steps)   # each call is one launch: this is also the launch's average duration
    # Untimed: the wire byte count (one device atomic per record).
    hc.hc_compressed_allreduce(send, recv, n, ws, wire)
    torch.cuda.synchronize()
    wire_bytes = int(wire.item())
    # The step-per-launch schedule beside it.
    key = "HC_CHAIN_MAX_BYTES"
    old = os.environ.get(key)
    os.environ[key] = "0"
    try:
        for _ in range(warmup):
            call()
        ms_steps = timed_ms(call, args.steps)
    finally:
        if old is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = old
    evsets = [hc.StepEvents.for_steps(steps, mode=1) for _ in range(args.steps)]
    for k in range(args.steps):
        hc.hc_compressed_allreduce(send, recv, n, ws, step_events=evsets[k])
    torch.cuda.synchronize()
    chunk = hc.hc_chunk_elems(n, 0.01, hc.HC_BLOCK_ELEMS)
    L = n // R
    nchunks = -(-L // chunk)
    framing = 0
    for c in range(nchunks):
        ln = min(chunk, L - c * chunk)
        framing += 32 + 16 * (-(-8 * (-(-ln // hc.HC_BLOCK_ELEMS)) // 16))
    framing *= R * 2 * (R - 1)
    rec_bytes = wire_bytes - framing
    alg = 4 * R * n + 2 * rec_bytes     # every rank's input read and output written once, every record written and read once
    parts = {"first": [], "rs": [], "ag": []}
    for ev in evsets:
        d = ev.elapsed_ms()
        parts["first"].append(d[0])
        parts["rs"] += d[1:R]
        parts["ag"] += d[R:]
    raw_wire = 2 * (R - 1) * n * 2
    rs_ms = sum(parts["rs"]) / len(parts["rs"])
    rec_hop = rec_bytes / (2 * (R - 1))           # records moved by one hop, all ranks
    extra = {"roofline": roofline_obj("car_chain_kernel (the whole allreduce in one launch: every codec block "
                                      "through every hop)", alg, ms,
                                      load_traffic("car_chain", "compressed", CODEC_FILES),
                                      "average over the timed back-to-back calls (HIP events around them); "
                                      "each call is that one launch")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 23
        xs = [inputs.host_bits(t[:m]) for t in send]
        extra["cpu_baseline"] = oracle_timed(lambda: oracle.compressed_allreduce(xs), 2 * m,
                                             f"oracle compressed allreduce of the first {m} elements of every rank "
                                             "(algbw: elements x 2 bytes per second)")
    return {**extra, "metric": "Compressed ring AllReduce algbw and achieved HBM GB/s, R=8, 2^25 bf16",
            "value": round(n * 2 / (ms / 1e3) / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"fused compressed ring allreduce, R={R} x {n} bf16 N(0,1e-3), chunk {chunk}"},
            "schedule": "one launch",
            "hbm_gbps": round(alg / (ms / 1e3) / 1e9, 1), "hbm_frac_of_peak": round(alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
            "alg_bytes": alg, "wire_bytes": wire_bytes, "wire_ratio": round(wire_bytes / raw_wire, 5),
            "step_schedule": {
                "ms_per_call": round(ms_steps, 5),
                "hbm_frac_of_peak": round(alg / (ms_steps / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
                "first_ms": round(sum(parts["first"]) / len(parts["first"]), 5),
                "rs_step_ms": round(rs_ms, 5),
                "ag_step_ms": round(sum(parts["ag"]) / len(parts["ag"]), 5),
                "car_rs_roofline": roofline_obj("car_rs_kernel (one reduce-scatter hop: decode, hop, encode)",
                                                int(2 * n + 2 * rec_hop), rs_ms, None,
                                                "mean reduce-scatter step by its kernel's start and end stamps "
                                                "(HIP events; the last step also writes the output)")}}


def bench_fused_sgd(args):
    """The allreduce of R=8 x 2^26 bf16 gradients fused with an SGD update of
    replicated bf16 weights (hc_allreduce_sgd), next to the unfused sequence:
    hc_allreduce of the gradients, then every rank updating its whole buffer
    (torch's w.sub_(g, alpha=lr); rounding aside, the same arithmetic)."""
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, n, lr = 8, 1 << 26, 0.01
    grads = inputs.ring_inputs_cuda("ring_bf16", R, n)
    w0 = inputs.normal_bf16_cuda("fused_sgd", 0, n, 1.0)
    weights = [w0.clone() for _ in range(R)]
    sums = [torch.empty_like(g) for g in grads]

    def fused():
        hc.hc_allreduce_sgd(grads, weights, lr)

    def unfused():
        hc.hc_allreduce(grads, sums)
        for w, g in zip(weights, sums):
            w.sub_(g, alpha=lr)

    for _ in range(args.warmup):
        fused()
        unfused()
    ms = timed_ms(fused, args.steps)
    ms_unfused = timed_ms(unfused, args.steps)
    steps = hc.hc_step_count(hc.HC_OP_ALLREDUCE, R)
    evsets = [hc.StepEvents.for_steps(steps, mode=1) for _ in range(args.steps)]
    for k in range(args.steps):
        hc.hc_allreduce_sgd(grads, weights, lr, step_events=evsets[k])
    torch.cuda.synchronize()
    last = [ev.elapsed_ms()[R - 2] for ev in evsets]
    # bytes: R-2 plain reduce steps (read 2, write 1), the fused step (read 3,
    # write 2: the new weights in place and into the next rank), R-2 copy
    # steps (read 1, write 1), every one over n bf16 elements
    alg = 2 * n * (3 * (R - 2) + 5 + 2 * (R - 2))
    alg_unfused = 2 * n * (3 * (R - 1) + 2 * (R - 1)) + 2 * n * R * 3
    last_ms = sum(last) / len(last)
    extra = {"roofline": roofline_obj("step_kernel<2,sgd-send> (the last reduce-scatter step with the update)", 10 * n,
                                      last_ms, None, "the step's kernel start and end stamps (HIP events)")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 24
        gs = [inputs.host_bits(t[:m]) for t in grads]
        wh = [inputs.host_bits(w0[:m])] * R
        extra["cpu_baseline"] = oracle_timed(lambda: oracle.allreduce_sgd(gs, wh, lr), 2 * m,
                                             f"oracle allreduce + SGD of the first {m} elements of every rank "
                                             "(algbw: elements x 2 bytes per second)")
    return {**extra, "metric": "Allreduce fused with an SGD update: algbw and achieved HBM GB/s, R=8, 2^26 bf16",
            "value": round(n * 2 / (ms / 1e3) / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"hc_allreduce_sgd, R={R} x {n} bf16 gradients N(0,1e-3) with 1% zeros, "
                                   f"replicated bf16 weights N(0,1), lr={lr}"},
            "hbm_gbps": round(alg / (ms / 1e3) / 1e9, 1),
            "hbm_frac_of_peak": round(alg / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4), "alg_bytes": alg,
            "fused_step_ms": round(sum(last) / len(last), 5),
            "fused_step_gbps": round(10 * n / (sum(last) / len(last) / 1e3) / 1e9, 1),
            "unfused_ms": round(ms_unfused, 5), "unfused_alg_bytes": alg_unfused,
            "speedup_vs_unfused": round(ms_unfused / ms, 3)}


def bench_contention(args):
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, n = 8, 1 << 28
    L = n // R
    send = inputs.ring_inputs_cuda("contention", R, n)
    recv = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(inputs.seed64("contention", 100))
    A = torch.randn(8192, 8192, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    Bm = torch.randn(8192, 8192, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    C = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    # The GEMM runs on a non-blocking stream: a CU-masked HIP stream is a
    # blocking stream, which the legacy default stream would serialize with.
    main = torch.cuda.Stream()
    rs_bytes = 3 * 2 * n * (R - 1)

    def gemm_alone(iters, stream=None):
        st = stream if stream is not None else main
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            for _ in range(2):
                torch.matmul(A, Bm, out=C)
        e0.record(st)
        with torch.cuda.stream(st):
            for _ in range(iters):
                torch.matmul(A, Bm, out=C)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    with torch.cuda.stream(main):
        for _ in range(3):
            torch.matmul(A, Bm, out=C)
    torch.cuda.synchronize()
    t_gemm = gemm_alone(10)

    def measure(op, side, cu_used, nbytes, prefix, gemm_stream=None, t_gemm_ref=None):
        """`op(stream)` alone on `side`, then again while the GEMM loops on the
        main stream for as long as it runs."""
        for _ in range(2):
            op(side)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        op(side)
        e1.record(side)
        torch.cuda.synchronize()
        t_alone = e0.elapsed_time(e1)
        gs = gemm_stream if gemm_stream is not None else main
        tg = t_gemm_ref if t_gemm_ref is not None else t_gemm
        iters = max(4, int(t_alone / tg) + 2)
        base = torch.cuda.Event(enable_timing=True)
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        base.record(gs)
        side.wait_event(base)
        r0.record(side)
        op(side)
        r1.record(side)
        ge[0].record(gs)
        with torch.cuda.stream(gs):
            for i in range(iters):
                torch.matmul(A, Bm, out=C)
                ge[i + 1].record(gs)
        torch.cuda.synchronize()
        gt = [base.elapsed_time(e) for e in ge]
        t0, t1 = base.elapsed_time(r0), base.elapsed_time(r1)
        overl = [gt[i + 1] - gt[i] for i in range(iters) if gt[i] < t1 and gt[i + 1] > t0]
        t_gemm_conc = median(overl) if overl else float("nan")
        rate = contention_rate([(gt[i], gt[i + 1]) for i in range(iters)], [(t0, t1, cu_used)], N_CU)
        return {f"{prefix}_alone_ms": round(t_alone, 4), f"{prefix}_concurrent_ms": round(t1 - t0, 4),
                f"{prefix}_alone_gbps": round(nbytes / t_alone / 1e6, 1),
                f"{prefix}_concurrent_gbps": round(nbytes / (t1 - t0) / 1e6, 1),
                "gemm_alone_ms": round(tg, 4), "gemm_concurrent_ms": round(t_gemm_conc, 4),
                "gemm_slowdown": round(t_gemm_conc / tg - 1, 4),
                "contention_rate": round(rate, 5) if rate is not None else None}

    rows = []
    for k in (8, 16, 32, 0):
        handle = hc.hc_stream_create_cu_budget(k) if k else None
        side = torch.cuda.ExternalStream(handle) if k else torch.cuda.Stream()
        row = {"op": "reduce_scatter", "cu_budget": k if k else "all"}
        rs_op = (lambda st, k=k: hc.hc_reduce_scatter(send, recv, L, ws, cu_budget=k, stream=st))
        row.update(measure(rs_op, side, k if k else N_CU, rs_bytes, "rs"))
        if k:
            # The GEMM confined to the other N_CU - k CUs: alone, and beside the
            # reduce-scatter.  Alone it shows what losing k CUs costs; beside
            # it, whatever is left is memory-system contention, since the two
            # share no CU (hc_cu_census measures the split).
            ch = hc.hc_stream_create_cu_range(k, N_CU - k)
            comp = torch.cuda.ExternalStream(ch)
            t_comp = gemm_alone(10, comp)
            cm = measure(rs_op, side, k, rs_bytes, "rs", gemm_stream=comp, t_gemm_ref=t_comp)
            row["complement"] = {"gemm_alone_ms": round(t_comp, 4),
                                 "gemm_alone_slowdown_vs_all_cus": round(t_comp / t_gemm - 1, 4),
                                 "gemm_concurrent_ms": cm["gemm_concurrent_ms"],
                                 "gemm_slowdown_vs_complement_alone": cm["gemm_slowdown"],
                                 "gemm_slowdown_vs_all_cus": round(cm["gemm_concurrent_ms"] / t_gemm - 1, 4),
                                 "rs_concurrent_gbps": cm["rs_concurrent_gbps"],
                                 "contention_rate": cm["contention_rate"]}
            del comp
            hc.hc_stream_destroy(ch)
        rows.append(row)
        if k:
            del side
            hc.hc_stream_destroy(handle)
    full = rows[-1]
    extra = {"roofline": roofline_obj("step_kernel<reduce> (reduce-scatter alone on all CUs, mean of its launches)",
                                      3 * 2 * n, full["rs_alone_ms"] / (R - 1),
                                      load_traffic("reduce_step", "contention", RING_FILES),
                                      "one reduce-scatter of R-1 launches by HIP events, divided by R-1")}
    if not args.no_cpu_baseline:
        import oracle

        m = 1 << 24
        xs = [inputs.host_bits(t[:m]) for t in send]
        extra["cpu_baseline"] = oracle_timed(lambda: oracle.reduce_scatter_ring(xs), 3 * 2 * m * (R - 1),
                                             f"oracle reduce-scatter of the first {m} elements of every rank "
                                             "(algorithmic bytes per second, as the GPU rows)")
    # The all-gather that follows this reduce-scatter (R slices of L -> R
    # outputs of n), on copy kernels and on the DMA copy engines (the offload
    # of "HOCCL ...", section 2), measured by dma_contention in a process of
    # its own: inside this torch process the HIP runtime bundled with the
    # wheel serves hipMemcpyDeviceToDeviceNoCU with blit kernels on the CUs.
    del send, recv, ws
    torch.cuda.empty_cache()
    tool = os.path.join(ROOT, "measure", "dma_contention")
    try:
        r = subprocess.run([tool, "bench"], capture_output=True, text=True, timeout=600)
        ag = json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else {"error": r.stderr[-2000:]}
    except (OSError, ValueError, subprocess.TimeoutExpired) as exc:
        ag = {"error": repr(exc)}
    return {"metric": "Reduce-scatter under a CU budget beside a bf16 GEMM: contention rate, GEMM slowdown, RS GB/s",
            "value": rows[0]["rs_concurrent_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": 1, "warmup": 2,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"R={R} reduce-scatter of {R} x {n} bf16 N(0,1e-3) on a CU-masked side stream, "
                                   "main stream torch.matmul 8192^3 bf16; then the matching all-gather "
                                   f"({R} x {L} -> {R} x {n}) on CU copy kernels and on the DMA copy engines"},
            "gemm_tflops_alone": round(2 * 8192 ** 3 / (t_gemm / 1e3) / 1e12, 1), "rows": rows,
            "all_gather": ag, **extra}


def bench_hop_sizes(args):
    """The reduce-scatter hop (R=8 bf16, all CUs) at 2^24..2^28 elements per
    rank, per ring step, under each store policy and cache state:
      - policy "auto" (the library's choice), "cached" (2 vectors per lane,
        ordinary stores) and "stream" (1 vector per lane, non-temporal
        stores), forced through HC_STREAM_STORE_MIN_BYTES;
      - "scrub": a 2 GiB read-modify-write before each call evicts the
        Infinity Cache, so the first step starts cold;
      - "rotate K" (2^26 only): K sets of buffers used in turn, so a call's
        inputs were last touched K calls earlier.
    Step 0 reads only the inputs; every later step also reads the partial
    sums the step before it wrote (the reduce-scatter's workspace)."""
    import statistics

    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, es = 8, 2
    steps = hc.hc_step_count(hc.HC_OP_REDUCE_SCATTER, R)
    iters = max(args.steps, 2)
    scrub = torch.zeros(1 << 29, dtype=torch.float32, device="cuda")

    def make(n, seed):
        send = [inputs.normal_bf16_cuda("contention", 1000 * seed + r, n, 1e-3) for r in range(R)]
        recv = [torch.empty(n // R, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc.HC_BF16), dtype=torch.uint8,
                         device="cuda")
        return send, recv, ws

    def run(sets, n, flush):
        for k in range(args.warmup):
            s, r, w = sets[k % len(sets)]
            hc.hc_reduce_scatter(s, r, n // R, w)
        evs = [hc.StepEvents.for_steps(steps, mode=1) for _ in range(iters)]
        for k in range(iters):
            s, r, w = sets[k % len(sets)]
            if flush:
                scrub.add_(1.0)
            hc.hc_reduce_scatter(s, r, n // R, w, step_events=evs[k])
        torch.cuda.synchronize()
        d = [e.elapsed_ms() for e in evs]
        per = [statistics.median(x[i] for x in d) for i in range(steps)]
        b = 3 * es * n
        return {"step_us": [round(t * 1e3, 2) for t in per],
                "first_step_gbps": round(b / (per[0] / 1e3) / 1e9),
                "later_steps_gbps": round(b / (statistics.mean(per[1:]) / 1e3) / 1e9)}

    env_key = "HC_STREAM_STORE_MIN_BYTES"
    old = os.environ.get(env_key)
    rows = []
    try:
        for lg in (24, 25, 26, 27, 28):
            n = 1 << lg
            bufs = [make(n, lg)]
            for policy, val in (("auto", None), ("cached", str(1 << 62)), ("stream", "0")):
                if val is None:
                    os.environ.pop(env_key, None)
                else:
                    os.environ[env_key] = val
                rows.append({"log2_elems_per_rank": lg, "policy": policy, "scrub": False, **run(bufs, n, False)})
                if policy == "auto":
                    rows.append({"log2_elems_per_rank": lg, "policy": policy, "scrub": True, **run(bufs, n, True)})
            del bufs
            torch.cuda.empty_cache()
        os.environ.pop(env_key, None)
        n = 1 << 26
        sets = [make(n, 40 + k) for k in range(8)]
        for K in (1, 2, 4, 8):
            rows.append({"log2_elems_per_rank": 26, "policy": "auto", "rotate": K, **run(sets[:K], n, False)})
        del sets
    finally:
        if old is None:
            os.environ.pop(env_key, None)
        else:
            os.environ[env_key] = old
    auto28 = next(r for r in rows if r["log2_elems_per_rank"] == 28 and r["policy"] == "auto" and not r.get("scrub"))
    return {"metric": "reduce-scatter hop GB/s by operand size, store policy and cache state (R=8 bf16)",
            "value": auto28["later_steps_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": iters,
            "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "reduce-scatter of R=8 x 2^24..2^28 bf16 N(0,1e-3), all CUs; value: 2^28, "
                                   "library policy, steps after the first"},
            "bytes_per_step": "3 x 2 bytes x elements per rank (2 reads, 1 write per element of the step)",
            "rows": rows}

def bench_compressed_schedules(args):
    """The compressed allreduce (R = 2, 4, 8 bf16 N(0,1e-3), 2^18..2^25
    elements per rank) under its two schedules, forced through
    HC_CHAIN_MAX_BYTES: one launch per ring step ("steps"), or one launch in
    which each codec block of each slice goes through every hop ("one
    launch"); and with the variable unset ("auto", the library's default,
    which is one launch).
    Each call is timed alone by two HIP events; the median over the calls is
    reported.  The wire bytes of the two schedules are checked equal."""
    import statistics

    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    key = "HC_CHAIN_MAX_BYTES"
    old = os.environ.get(key)
    iters = max(args.steps, 3)
    rows = []
    try:
        for R in (2, 4, 8):
            for lg in (18, 20, 21, 22, 23, 24, 25):
                n = 1 << lg
                send = inputs.ring_inputs_cuda("compressed", R, n)
                recv = [torch.empty_like(t) for t in send]
                ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_COMPRESSED_ALLREDUCE, n, R), dtype=torch.uint8,
                                 device="cuda")
                slice_len = -(-n // R)
                row = {"R": R, "log2_elems_per_rank": lg, "grid": R * -(-slice_len // hc.HC_BLOCK_ELEMS)}
                wires = {}
                for name, val in (("steps", "0"), ("one_launch", str(1 << 62)), ("auto", None)):
                    if val is None:
                        os.environ.pop(key, None)
                    else:
                        os.environ[key] = val
                    wire = torch.zeros(1, dtype=torch.int64, device="cuda")
                    for _ in range(args.warmup):
                        hc.hc_compressed_allreduce(send, recv, n, ws)
                    hc.hc_compressed_allreduce(send, recv, n, ws, wire)
                    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                           for _ in range(iters)]
                    for a, b in evs:
                        a.record()
                        hc.hc_compressed_allreduce(send, recv, n, ws)
                        b.record()
                    torch.cuda.synchronize()
                    row[name + "_us"] = round(statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3, 1)
                    wires[name] = int(wire.item())
                if len(set(wires.values())) != 1:
                    raise RuntimeError(f"wire bytes differ between schedules: {wires}")
                row["one_launch_over_steps"] = round(row["one_launch_us"] / row["steps_us"], 3)
                rows.append(row)
                del send, recv, ws
                torch.cuda.empty_cache()
    finally:
        if old is None:
            os.environ.pop(key, None)
        else:
            os.environ[key] = old
    r8 = next(r for r in rows if r["R"] == 8 and r["log2_elems_per_rank"] == 22)
    return {"metric": "compressed allreduce time by schedule (R=2, 4, 8 bf16, 2^18..2^25 elements per rank)",
            "value": r8["auto_us"], "unit": "us", "n_gpus": 1, "steps": iters, "warmup": args.warmup,
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "compressed allreduce of R x n bf16 N(0,1e-3), chunk 1%; value: R=8 x 2^22, "
                                   "the library's schedule"},
            "rows": rows}

def bench_rs_budget(args):
    """The contention test's reduce-scatter (R=8 x 2^28 bf16, N(0,1e-3))
    without the GEMM: on a k-CU stream (hc_stream_create_cu_budget) for
    k = 8, 16, 32, and on all CUs, each timed alone by HIP events on its
    stream.  The run the CU-occupancy and traffic counters are taken on."""
    import torch

    from collective_communication_amd import binding as hc
    from collective_communication_amd import inputs

    R, n = 8, 1 << 28
    L = n // R
    send = inputs.ring_inputs_cuda("contention", R, n)
    recv = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
    ws = torch.empty(hc.hc_workspace_bytes(hc.HC_OP_REDUCE_SCATTER, n, R, hc.HC_BF16), dtype=torch.uint8,
                     device="cuda")
    rs_bytes = 3 * 2 * n * (R - 1)
    rows = []
    for k in (8, 16, 32, 0):
        handle = hc.hc_stream_create_cu_budget(k) if k else None
        side = torch.cuda.ExternalStream(handle) if k else torch.cuda.Stream()
        for _ in range(args.warmup):
            hc.hc_reduce_scatter(send, recv, L, ws, cu_budget=k, stream=side)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(args.steps):
            hc.hc_reduce_scatter(send, recv, L, ws, cu_budget=k, stream=side)
        e1.record(side)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        rows.append({"cu_budget": k if k else "all", "rs_ms": round(ms, 4),
                     "rs_gbps": round(rs_bytes / (ms / 1e3) / 1e9, 1)})
        del side
        if k:
            hc.hc_stream_destroy(handle)
    return {"metric": "reduce-scatter GB/s on k CUs (R=8 x 2^28 bf16, no concurrent GEMM)",
            "value": rows[0]["rs_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"R={R} reduce-scatter of {R} x {n} bf16 N(0,1e-3) on a k-CU stream; value: k = 8"},
            "bytes_per_call": rs_bytes, "rows": rows}

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ring_bf16",
                    choices=["ring_bf16", "ring_f32", "ring_bf16_carry", "codec", "compressed", "contention",
                             "fused_sgd", "table_scope", "entropy", "hop_sizes", "rs_budget",
                             "compressed_schedules"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26,
                    help="elements per rank the oracle baseline runs on (default: the whole workload)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the ring is emulated with all R ranks resident on one GPU; "
                                   "runs across several GPUs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.workload in ("ring_bf16", "ring_f32"):
        line = bench_ring(args, args.workload)
    elif args.workload == "ring_bf16_carry":
        line = bench_ring_carry(args)
    elif args.workload == "codec":
        line = bench_codec(args)
    elif args.workload == "compressed":
        line = bench_compressed(args)
    elif args.workload == "fused_sgd":
        line = bench_fused_sgd(args)
    elif args.workload == "table_scope":
        line = bench_table_scope(args)
    elif args.workload == "entropy":
        line = bench_entropy(args)
    elif args.workload == "hop_sizes":
        line = bench_hop_sizes(args)
    elif args.workload == "rs_budget":
        line = bench_rs_budget(args)
    elif args.workload == "compressed_schedules":
        line = bench_compressed_schedules(args)
    else:
        line = bench_contention(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
