"""CPU lint over the HIP sources.

The cross-lane read builtins (readlane, readfirstlane) return a signed int.
Widened into a 64-bit offset without going back to unsigned first, a word
with bit 31 set sign-extends into a wild address: a kernel of this library
once faulted exactly so on a stream past 2 GB.  Kernels therefore read lanes
only through the unsigned helpers defined next to the other device helpers;
this test keeps every other use of the builtins out of the sources, and
checks the helpers themselves return unsigned values."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "collective_communication_amd")
HELPERS = os.path.join(PKG, "csrc", "common.hpp")
BUILTIN = re.compile(r"__builtin_amdgcn_read(first)?lane\s*\(")


def sources():
    for d, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".hip", ".hpp", ".cpp", ".h")):
                yield os.path.join(d, f)


def code_lines(path):
    """Lines with // comments removed (the sources use no block comments in code)."""
    with open(path) as f:
        for i, ln in enumerate(f, 1):
            yield i, ln.split("//", 1)[0]


def test_no_raw_lane_read_builtins_outside_the_helpers():
    bad = []
    for p in sources():
        if p == HELPERS:
            continue
        for i, ln in code_lines(p):
            if BUILTIN.search(ln):
                bad.append(f"{os.path.relpath(p, ROOT)}:{i}: {ln.strip()}")
    assert not bad, "raw cross-lane read builtins (use lane_read / first_lane_read):\n" + "\n".join(bad)


def test_lane_read_helpers_return_unsigned():
    text = open(HELPERS).read()
    for name, ret in (("lane_read", "uint32_t"), ("first_lane_read", "uint32_t"), ("lane_read64", "uint64_t")):
        m = re.search(r"__device__ __forceinline__ (\w+) " + name + r"\(", text)
        assert m and m.group(1) == ret, f"{name} must return {ret}"
        body = text[m.end():text.index("}", m.end())]
        if name != "lane_read64":
            assert f"return ({ret})__builtin_amdgcn_read" in body, f"{name} must cast the builtin's int to {ret}"


def test_lint_catches_a_raw_use(tmp_path):
    """The pattern itself: a raw use in a line of code is found, one in a
    comment is not."""
    assert BUILTIN.search("  const uint64_t off = __builtin_amdgcn_readfirstlane(lo);")
    assert BUILTIN.search("x = __builtin_amdgcn_readlane (v, 3);")
    assert not BUILTIN.search("  // __builtin_amdgcn_readlane(v, 3)".split("//", 1)[0])
