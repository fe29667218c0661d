"""Plain single-threaded CPU oracle for the emulated ring AllReduce and the
HCZ1 lossless bf16 codec.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this package; the product path
(``collective_communication_amd``) never imports it and shares no code with it.

The arithmetic lives in ``hc_oracle.c`` (built with gcc, no fast-math, no
FP contraction); this module only marshals numpy arrays through ctypes.  Each
function's C docstring cites the passage it follows:

* the ring (reduce-scatter, all-gather, allreduce) follows the AllReduce =
  ReduceScatter then AllGather split of "Breaking the computation and
  communication abstraction barrier in distributed machine learning
  workloads" (section "The idea") and the primitives/chunk terms of "ResCCL:
  Resource-Efficient Scheduling for Collective Communication" (section 1);
* the codec follows "CCCL: In-GPU Compression-Coupled Collective
  Communication", sections 4.1, 4.3, 4.4 and 5 ("Handling data alignment");
* the entropy-coded variant (``hce_oracle.c``) codes the exponent with a
  per-block canonical Huffman code instead (CCCL sections 4.1 and 6.5);
* the contention rate follows "HOCCL: Offloading Collective Communication from
  GPU Cores to Accelerate Distributed Training", section 2 (its formula is
  lost from the page; the reading is stated in ``hc_oracle.c``).

Parity unpinned: the absolute throughput of anything (the pages print no
figure for this hardware), and fidelity of the contention formula to HOCCL's
lost equation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "hc_oracle.c"), os.path.join(_HERE, "hce_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle_hc.so")

F32 = 0
BF16 = 1
OK = 0
INVALID = 1
CAPACITY = 3
CORRUPT = 4
BLOCK = 16384
OP_RRC = 1
OP_COPY = 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE adds: no fast-math, no contraction)."""
    stale = not os.path.exists(_LIB_PATH) or any(
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(src) for src in _SRCS)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Task(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32), ("step", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("op", ctypes.c_int32), ("slice", ctypes.c_int32),
                ("off", ctypes.c_uint64), ("len", ctypes.c_uint64)]


class _Plan(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("b", ctypes.c_int32), ("m", ctypes.c_uint32),
                ("n_esc", ctypes.c_uint32), ("rec_bytes", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        S = ctypes.c_size_t
        PP = ctypes.POINTER(ctypes.c_void_p)
        L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_f32.restype = ctypes.c_float
        L.or_f32_to_bf16.argtypes = [ctypes.c_uint32]
        L.or_f32_to_bf16.restype = ctypes.c_uint16
        L.or_hop_f32.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.or_hop_f32.restype = ctypes.c_uint32
        L.or_hop_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.or_hop_bf16.restype = ctypes.c_uint16
        L.or_sgd_f32.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_float]
        L.or_sgd_f32.restype = ctypes.c_uint32
        L.or_sgd_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_float]
        L.or_sgd_bf16.restype = ctypes.c_uint16
        L.or_allreduce_sgd.argtypes = [PP, PP, PP, S, ctypes.c_int, ctypes.c_int, ctypes.c_float]
        L.or_allreduce_sgd.restype = ctypes.c_int
        L.or_slice_len.argtypes = [S, ctypes.c_int]
        L.or_slice_len.restype = S
        L.or_chunk_elems.argtypes = [S, S]
        L.or_chunk_elems.restype = S
        L.or_ring_tasks.argtypes = [ctypes.c_int, S, S, ctypes.POINTER(_Task), S]
        L.or_ring_tasks.restype = S
        for name in ("or_allreduce_fold",):
            getattr(L, name).argtypes = [PP, PP, S, ctypes.c_int, ctypes.c_int]
            getattr(L, name).restype = ctypes.c_int
        L.or_allreduce_fold_f32carry.argtypes = [PP, PP, S, ctypes.c_int]
        L.or_allreduce_fold_f32carry.restype = ctypes.c_int
        L.or_allreduce_fold_at.argtypes = [PP, S, ctypes.c_int, ctypes.c_int, P, S, P]
        L.or_allreduce_fold_at.restype = ctypes.c_int
        for name in ("or_allreduce_ring", "or_reduce_scatter_ring", "or_all_gather_ring"):
            getattr(L, name).argtypes = [PP, PP, S, ctypes.c_int, ctypes.c_int, S]
            getattr(L, name).restype = ctypes.c_int
        L.or_compress_bound.argtypes = [S]
        L.or_compress_bound.restype = S
        L.or_plan_block.argtypes = [P, S, ctypes.POINTER(_Plan)]
        L.or_plan_block.restype = ctypes.c_int
        L.or_compress.argtypes = [P, S, P, S]
        L.or_compress.restype = S
        L.or_compress_scoped.argtypes = [P, S, P, S, S]
        L.or_compress_scoped.restype = S
        L.or_decompress.argtypes = [P, S, P, S]
        L.or_decompress.restype = ctypes.c_int
        L.or_compressed_allreduce.argtypes = [PP, PP, S, ctypes.c_int, S,
                                              ctypes.POINTER(ctypes.c_uint64)]
        L.or_compressed_allreduce.restype = ctypes.c_int
        L.or_f32_to_bf16_array.argtypes = [P, P, S]
        L.or_f32_to_bf16_array.restype = None
        L.or_hop_bf16_array.argtypes = [P, P, P, S]
        L.or_hop_bf16_array.restype = None
        L.or_hop_f32_array.argtypes = [P, P, P, S]
        L.or_hop_f32_array.restype = None
        L.or_huff_lengths.argtypes = [P, ctypes.c_int, P]
        L.or_huff_lengths.restype = ctypes.c_int
        L.or_huff_codes.argtypes = [P, ctypes.c_int, P]
        L.or_huff_codes.restype = None
        L.or_hce_bound.argtypes = [S]
        L.or_hce_bound.restype = S
        L.or_hce_compress.argtypes = [P, S, P, S]
        L.or_hce_compress.restype = S
        L.or_hce_decompress.argtypes = [P, S, P, S]
        L.or_hce_decompress.restype = ctypes.c_int
        L.or_hce_plan_block.argtypes = [P, S, P]
        L.or_hce_plan_block.restype = ctypes.c_int
        D = ctypes.POINTER(ctypes.c_double)
        L.or_contention_rate.argtypes = [D, D, S, D, D, D, S, ctypes.c_double]
        L.or_contention_rate.restype = ctypes.c_double
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint32 or a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes fp32 (float32/uint32) or bf16 bit patterns (uint16), got {a.dtype}")


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def _check_same(xs):
    xs = [np.ascontiguousarray(x) for x in xs]
    if not xs:
        raise ValueError("need at least one rank")
    for x in xs:
        if x.dtype != xs[0].dtype or x.shape != xs[0].shape or x.ndim != 1:
            raise ValueError("all ranks need 1-D buffers of one dtype and length")
    return xs


# ----------------------------------------------------------------------------
# scalar rules
# ----------------------------------------------------------------------------

def f32_to_bf16(bits: int) -> int:
    return int(lib().or_f32_to_bf16(bits & 0xFFFFFFFF))


def f32_to_bf16_array(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(bits.size, dtype=np.uint16)
    lib().or_f32_to_bf16_array(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def hop_bf16_array(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(a.size, dtype=np.uint16)
    lib().or_hop_bf16_array(a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size)
    return out


def hop_f32_array(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a).view(np.uint32)
    b = np.ascontiguousarray(b).view(np.uint32)
    out = np.empty(a.size, dtype=np.uint32)
    lib().or_hop_f32_array(a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size)
    return out


def hop_bf16(a: int, b: int) -> int:
    return int(lib().or_hop_bf16(a, b))


def hop_f32(a: int, b: int) -> int:
    return int(lib().or_hop_f32(a, b))


# ----------------------------------------------------------------------------
# ring
# ----------------------------------------------------------------------------

def slice_len(n: int, R: int) -> int:
    return int(lib().or_slice_len(n, R))


def chunk_elems(n: int, align: int = 1024) -> int:
    return int(lib().or_chunk_elems(n, align))


def ring_tasks(R: int, n: int, chunk: int):
    """Task list as a structured numpy array with fields src, dst, step, chunk, op, slice, off, len."""
    cnt = int(lib().or_ring_tasks(R, n, chunk, None, 0))
    buf = (_Task * max(cnt, 1))()
    lib().or_ring_tasks(R, n, chunk, buf, cnt)
    dt = np.dtype([("src", "<i4"), ("dst", "<i4"), ("step", "<i4"), ("chunk", "<i4"),
                   ("op", "<i4"), ("slice", "<i4"), ("off", "<u8"), ("len", "<u8")])
    return np.frombuffer(bytes(buf)[: cnt * ctypes.sizeof(_Task)], dtype=dt).copy()


def allreduce_fold(xs):
    """Closed-form ring allreduce; returns one array (every rank holds a copy)."""
    xs = _check_same(xs)
    R, n = len(xs), xs[0].size
    outs = [np.empty_like(xs[0]) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    rc = lib().or_allreduce_fold(xp, op, n, _dtype_code(xs[0]), R)
    if rc != OK:
        raise ValueError(f"or_allreduce_fold status {rc}")
    return outs


def sgd_f32(w: int, g: int, lr: float) -> int:
    return int(lib().or_sgd_f32(w, g, lr))


def sgd_bf16(w: int, g: int, lr: float) -> int:
    return int(lib().or_sgd_bf16(w, g, lr))


def allreduce_sgd(grads, weights, lr: float):
    """Allreduce of the gradients fused with the update w - lr*g on each
    slice owner's weights; returns the R weight buffers after the call (all
    equal).  lr is taken as an fp32 value."""
    grads = _check_same(grads)
    weights = _check_same(weights)
    if weights[0].dtype != grads[0].dtype or weights[0].size != grads[0].size or len(weights) != len(grads):
        raise ValueError("grads and weights need one dtype, size and rank count")
    R, n = len(grads), grads[0].size
    outs = [np.empty_like(grads[0]) for _ in range(R)]
    gp, _k1 = _ptrs(grads)
    wp, _k2 = _ptrs(weights)
    op, _k3 = _ptrs(outs)
    rc = lib().or_allreduce_sgd(gp, wp, op, n, _dtype_code(grads[0]), R, lr)
    if rc != OK:
        raise ValueError(f"or_allreduce_sgd status {rc}")
    return outs


def allreduce_fold_f32carry(xs):
    """bf16 ring allreduce with fp32 partials and one final rounding (the
    fp32-carry reading); returns the R output arrays (all equal)."""
    xs = _check_same(xs)
    if xs[0].dtype != np.uint16:
        raise TypeError("the fp32-carry fold takes bf16 bit patterns (uint16)")
    R, n = len(xs), xs[0].size
    outs = [np.empty_like(xs[0]) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    rc = lib().or_allreduce_fold_f32carry(xp, op, n, R)
    if rc != OK:
        raise ValueError(f"or_allreduce_fold_f32carry status {rc}")
    return outs


def allreduce_fold_at(xs, idx):
    xs = _check_same(xs)
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    vals = np.empty(idx.size, dtype=xs[0].dtype)
    xp, _k = _ptrs(xs)
    rc = lib().or_allreduce_fold_at(xp, xs[0].size, _dtype_code(xs[0]), len(xs),
                                    idx.ctypes.data, idx.size, vals.ctypes.data)
    if rc != OK:
        raise ValueError(f"or_allreduce_fold_at status {rc}")
    return vals


def allreduce_ring(xs, chunk: int | None = None):
    """Step-simulated ring allreduce; returns the R output buffers."""
    xs = _check_same(xs)
    R, n = len(xs), xs[0].size
    if chunk is None:
        chunk = chunk_elems(n)
    outs = [np.zeros_like(xs[0]) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    rc = lib().or_allreduce_ring(xp, op, n, _dtype_code(xs[0]), R, chunk)
    if rc != OK:
        raise ValueError(f"or_allreduce_ring status {rc}")
    return outs


def reduce_scatter_ring(xs, chunk: int | None = None):
    xs = _check_same(xs)
    R, n = len(xs), xs[0].size
    if n % R:
        raise ValueError("reduce-scatter needs the buffer length to divide by R")
    recv = n // R
    if chunk is None:
        chunk = chunk_elems(n)
    outs = [np.zeros(recv, dtype=xs[0].dtype) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    rc = lib().or_reduce_scatter_ring(xp, op, recv, _dtype_code(xs[0]), R, chunk)
    if rc != OK:
        raise ValueError(f"or_reduce_scatter_ring status {rc}")
    return outs


def all_gather_ring(xs, chunk: int | None = None):
    xs = _check_same(xs)
    R, n = len(xs), xs[0].size
    if chunk is None:
        chunk = chunk_elems(n * R)
    outs = [np.zeros(n * R, dtype=xs[0].dtype) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    rc = lib().or_all_gather_ring(xp, op, n, _dtype_code(xs[0]), R, chunk)
    if rc != OK:
        raise ValueError(f"or_all_gather_ring status {rc}")
    return outs


# ----------------------------------------------------------------------------
# codec
# ----------------------------------------------------------------------------

def compress_bound(n: int) -> int:
    return int(lib().or_compress_bound(n))


def plan_block(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.uint16)
    p = _Plan()
    rc = lib().or_plan_block(v.ctypes.data, v.size, ctypes.byref(p))
    if rc != OK:
        raise ValueError(f"or_plan_block status {rc}")
    return {"mode": p.mode, "b": p.b, "m": p.m, "n_esc": p.n_esc, "rec_bytes": p.rec_bytes}


def compress(v: np.ndarray) -> bytes:
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cap = compress_bound(v.size)
    out = np.zeros(cap, dtype=np.uint8)
    sz = int(lib().or_compress(v.ctypes.data, v.size, out.ctypes.data, cap))
    if sz == 0:
        raise RuntimeError("oracle compress: capacity")
    return out[:sz].tobytes()


def compress_scoped(v: np.ndarray, group: int) -> bytes:
    """HCZ1 stream whose code tables are shared by groups of `group` full
    blocks (0: one table for the whole stream); group 1 is compress()."""
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cap = compress_bound(v.size)
    out = np.zeros(cap, dtype=np.uint8)
    sz = int(lib().or_compress_scoped(v.ctypes.data, v.size, out.ctypes.data, cap, group))
    if sz == 0:
        raise RuntimeError("oracle compress_scoped: capacity")
    return out[:sz].tobytes()


def decompress(stream: bytes, n: int):
    """Returns (status, array).  On a corrupt stream the array is all zero."""
    buf = np.frombuffer(stream, dtype=np.uint8).copy() if len(stream) else np.zeros(1, np.uint8)
    out = np.zeros(max(n, 1), dtype=np.uint16)
    rc = int(lib().or_decompress(buf.ctypes.data, len(stream), out.ctypes.data, n))
    return rc, out[:n]


# ----------------------------------------------------------------------------
# entropy-coded variant (HCE1)
# ----------------------------------------------------------------------------

def huff_lengths(counts, lmax: int = 12) -> np.ndarray:
    """Length-limited Huffman code lengths (uint8[256]) for 256 counts."""
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    if c.size != 256:
        raise ValueError("256 counts")
    out = np.zeros(256, dtype=np.uint8)
    lib().or_huff_lengths(c.ctypes.data, lmax, out.ctypes.data)
    return out


def huff_codes(lengths, lmax: int = 12) -> np.ndarray:
    """Canonical codes (uint32[256], right-aligned) for 256 code lengths."""
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(256, dtype=np.uint32)
    lib().or_huff_codes(ln.ctypes.data, lmax, out.ctypes.data)
    return out


def hce_bound(n: int) -> int:
    return int(lib().or_hce_bound(n))


def hce_plan_block(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.uint16)
    out = np.zeros(4, dtype=np.uint32)
    if lib().or_hce_plan_block(v.ctypes.data, v.size, out.ctypes.data) != 0:
        raise ValueError("block size")
    return {"mode": int(out[0]), "n_sym": int(out[1]), "n_words": int(out[2]), "rec_bytes": int(out[3])}


def hce_compress(v: np.ndarray) -> bytes:
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cap = hce_bound(v.size)
    out = np.zeros(cap, dtype=np.uint8)
    sz = int(lib().or_hce_compress(v.ctypes.data, v.size, out.ctypes.data, cap))
    if sz == 0:
        raise RuntimeError("oracle hce_compress: capacity")
    return out[:sz].tobytes()


def hce_decompress(stream: bytes, n: int):
    """Returns (status, array).  On a corrupt stream the array is all zero."""
    buf = np.frombuffer(stream, dtype=np.uint8).copy() if len(stream) else np.zeros(1, np.uint8)
    out = np.zeros(max(n, 1), dtype=np.uint16)
    rc = int(lib().or_hce_decompress(buf.ctypes.data, len(stream), out.ctypes.data, n))
    return rc, out[:n]


def compressed_allreduce(xs, chunk: int | None = None):
    """Returns (outputs, wire_bytes)."""
    xs = _check_same(xs)
    if xs[0].dtype != np.uint16:
        raise TypeError("compressed allreduce is bf16 only")
    R, n = len(xs), xs[0].size
    if chunk is None:
        chunk = chunk_elems(n, BLOCK)
    outs = [np.zeros_like(xs[0]) for _ in range(R)]
    xp, _k1 = _ptrs(xs)
    op, _k2 = _ptrs(outs)
    wire = ctypes.c_uint64(0)
    rc = lib().or_compressed_allreduce(xp, op, n, R, chunk, ctypes.byref(wire))
    if rc != OK:
        raise ValueError(f"or_compressed_allreduce status {rc}")
    return outs, int(wire.value)


# ----------------------------------------------------------------------------
# contention rate
# ----------------------------------------------------------------------------

def contention_rate(compute, comm, n_cu: float) -> float:
    """compute: list of (t0, t1); comm: list of (t0, t1, cus)."""
    D = ctypes.c_double
    c0 = (D * max(len(compute), 1))(*[a for a, _ in compute])
    c1 = (D * max(len(compute), 1))(*[b for _, b in compute])
    m0 = (D * max(len(comm), 1))(*[a for a, _, _ in comm])
    m1 = (D * max(len(comm), 1))(*[b for _, b, _ in comm])
    mc = (D * max(len(comm), 1))(*[c for _, _, c in comm])
    return float(lib().or_contention_rate(c0, c1, len(compute), m0, m1, mc, len(comm), n_cu))
