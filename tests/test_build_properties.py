"""CPU checks of properties of the device code that the tests on the GPU
would not catch, because a breach changes speed, not values.

The one-launch compressed allreduce (csrc/car_chain.hip) runs every hop of
a codec block in one loop.  Its file sets HC_CODEC_OPAQUE_TID before any
include, so that the codec helpers take their thread index through an opaque
read and no per-lane offset is held across the loop; without it the kernel
spills hundreds of bytes per lane.  Every other file keeps the plain read
(the opaque one slows the one-block encoders).  The second check compiles
the codec sources for gfx950 and reads the compiler's resource report: the
one-launch kernel within 64 VGPRs and a small spill, the one-block codec
kernels without scratch."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "collective_communication_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
MACRO = "HC_CODEC_OPAQUE_TID"


def code(path):
    with open(path) as f:
        return "\n".join(ln.split("//", 1)[0] for ln in f)


def test_only_the_chain_file_sets_the_opaque_index():
    setters = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp")) and re.search(r"#define\s+" + MACRO + r"\s+1", code(os.path.join(CSRC, f))):
            setters.append(f)
    assert setters == ["car_chain.hip"], setters


def test_chain_file_sets_it_before_any_include():
    text = code(os.path.join(CSRC, "car_chain.hip"))
    define = re.search(r"#define\s+" + MACRO + r"\s+1", text)
    first_include = re.search(r"#include", text)
    assert define and first_include and define.start() < first_include.start()


def test_headers_default_to_the_plain_read():
    text = code(os.path.join(CSRC, "codec.hpp"))
    assert re.search(r"#ifndef\s+" + MACRO + r"\s*\n\s*#define\s+" + MACRO + r"\s+0", text)
    # the two builds of the helpers must not share names
    assert "inline namespace HC_CODEC_TID_NS" in text


def resource_usage(src):
    cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-rdc",
           "--cuda-device-only", "-x", "hip", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    usage, name = {}, None
    for ln in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", ln)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]):\s+(\d+)", ln)
        if m and name:
            usage[name][m.group(1)] = int(m.group(2))
    return usage


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_register_budgets_of_the_codec_kernels():
    chain = resource_usage("car_chain.hip")
    k = [v for n, v in chain.items() if "car_chain_kernel" in n]
    assert len(k) == 1, list(chain)
    assert k[0]["VGPRs"] <= 64 and k[0]["ScratchSize [bytes/lane]"] <= 64, k[0]
    codec = resource_usage("codec_kernels.hip")
    one_block = {n: v for n, v in codec.items()
                 if re.search(r"(compress_kernel|decompress_kernel|car_first_kernel|car_rs_kernel|car_ag_kernel)", n)}
    assert len(one_block) >= 6, list(codec)
    for n, v in one_block.items():
        assert v["VGPRs"] <= 64 and v["ScratchSize [bytes/lane]"] == 0, (n, v)
