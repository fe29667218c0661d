"""ctypes binding of libhc (C ABI in include/hc.h), argument marshalling only.

Every function has the C name and order of arguments; torch device tensors
stand in for device pointers and torch streams for hipStream_t.  The only
logic here is turning tensors into pointers and sizes, checking that the
tensors are large enough for what the C call will touch, and raising
``HcError`` for a non-zero status.  There is no CPU fallback: when libhc.so
is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhc.so")

HC_SUCCESS = 0
HC_ERR_INVALID_ARGUMENT = 1
HC_ERR_UNSUPPORTED = 2
HC_ERR_INSUFFICIENT_CAPACITY = 3
HC_ERR_CORRUPT_STREAM = 4
HC_ERR_DEVICE = 5
HC_F32 = 0
HC_BF16 = 1
HC_OP_REDUCE_SCATTER = 0
HC_OP_COMPRESS = 1
HC_OP_COMPRESSED_ALLREDUCE = 2
HC_OP_ALLREDUCE = 3
HC_OP_ALL_GATHER = 4
HC_OP_COMPRESS_SCOPED = 5
HC_OP_COMPRESS_ENTROPY = 6
HC_OP_COMPRESS_STAGED = 7
HC_OP_ALLREDUCE_F32_CARRY = 8
HC_BLOCK_ELEMS = 16384
HC_MAX_RANKS = 64

EXPORTED = [
    "hc_allreduce", "hc_reduce_scatter", "hc_all_gather", "hc_compress_bound_bf16",
    "hc_compress_bf16", "hc_decompress_bf16", "hc_compressed_allreduce", "hc_workspace_bytes",
    "hc_stream_create_cu_budget", "hc_stream_destroy", "hc_chunk_elems", "hc_ring_tasks",
    "hc_status_string", "hc_last_error", "hc_version", "hc_step_count", "hc_allreduce_sgd",
    "hc_compress_bf16_scoped", "hc_compress_bf16_entropy", "hc_decompress_bf16_entropy",
    "hc_compress_bf16_staged", "hc_allreduce_bf16_f32carry", "hc_compress_bf16_noalloc", "hc_cu_census",
    "hc_stream_create_cu_range", "hc_copy_engine_available",
]


class HcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hc status {status}: {message}")
        self.status = status


class hc_opts_t(ctypes.Structure):
    _fields_ = [("chunk_fraction", ctypes.c_double), ("cu_budget", ctypes.c_int32),
                ("n_step_events", ctypes.c_int32), ("step_events", ctypes.c_void_p),
                ("copy_engine", ctypes.c_int32), ("step_event_mode", ctypes.c_int32)]


class hc_task_t(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("dst", ctypes.c_int32), ("step", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("op", ctypes.c_int32), ("slice", ctypes.c_int32),
                ("off", ctypes.c_uint64), ("len", ctypes.c_uint64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libhc.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(path)
    P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    PP = ctypes.POINTER(ctypes.c_void_p)
    O = ctypes.POINTER(hc_opts_t)
    L.hc_allreduce.argtypes = [PP, PP, S, I, I, O, P]
    L.hc_reduce_scatter.argtypes = [PP, PP, S, I, I, P, S, O, P]
    L.hc_all_gather.argtypes = [PP, PP, S, I, I, O, P]
    L.hc_allreduce_sgd.argtypes = [PP, PP, S, I, I, ctypes.c_float, O, P]
    L.hc_allreduce_bf16_f32carry.argtypes = [PP, PP, S, I, P, S, O, P]
    L.hc_compress_bound_bf16.argtypes = [S]
    L.hc_compress_bound_bf16.restype = S
    L.hc_compress_bf16.argtypes = [P, S, P, S, P, P, S, P]
    L.hc_compress_bf16_scoped.argtypes = [P, S, P, S, P, S, P, S, P]
    L.hc_compress_bf16_entropy.argtypes = [P, S, P, S, P, P, S, P]
    L.hc_compress_bf16_staged.argtypes = [P, S, P, S, P, P, S, P]
    L.hc_compress_bf16_noalloc.argtypes = [P, S, P, S, P, P]
    L.hc_decompress_bf16_entropy.argtypes = [P, S, P, S, P, P]
    L.hc_decompress_bf16.argtypes = [P, S, P, S, P, P]
    L.hc_compressed_allreduce.argtypes = [PP, PP, S, I, P, S, P, O, P]
    L.hc_workspace_bytes.argtypes = [I, S, I, I]
    L.hc_workspace_bytes.restype = S
    L.hc_stream_create_cu_budget.argtypes = [I, ctypes.POINTER(ctypes.c_void_p)]
    L.hc_stream_create_cu_range.argtypes = [I, I, ctypes.POINTER(ctypes.c_void_p)]
    L.hc_stream_destroy.argtypes = [P]
    L.hc_cu_census.argtypes = [P, I, I, P]
    L.hc_chunk_elems.argtypes = [S, ctypes.c_double, S]
    L.hc_chunk_elems.restype = S
    L.hc_ring_tasks.argtypes = [I, S, S, ctypes.POINTER(hc_task_t), S]
    L.hc_step_count.argtypes = [I, I]
    L.hc_step_count.restype = I
    L.hc_ring_tasks.restype = S
    for name in ("hc_allreduce", "hc_reduce_scatter", "hc_all_gather", "hc_allreduce_sgd",
                 "hc_allreduce_bf16_f32carry", "hc_compress_bf16",
                 "hc_compress_bf16_scoped", "hc_compress_bf16_entropy", "hc_compress_bf16_staged",
                 "hc_compress_bf16_noalloc", "hc_decompress_bf16",
                 "hc_decompress_bf16_entropy", "hc_compressed_allreduce", "hc_stream_create_cu_budget",
                 "hc_stream_destroy", "hc_cu_census", "hc_stream_create_cu_range"):
        getattr(L, name).restype = I
    L.hc_status_string.argtypes = [I]
    L.hc_status_string.restype = ctypes.c_char_p
    L.hc_last_error.argtypes = []
    L.hc_last_error.restype = ctypes.c_char_p
    L.hc_copy_engine_available.argtypes = []
    L.hc_copy_engine_available.restype = I
    L.hc_version.argtypes = []
    L.hc_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != HC_SUCCESS:
        L = load()
        raise HcError(status, f"{L.hc_status_string(status).decode()}: {L.hc_last_error().decode()}")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HC_F32
    if t.dtype == torch.bfloat16:
        return HC_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _current_stream_handle() -> int:
    # torch's raw stream query costs about a tenth of building a Stream object
    # (0.3 against 2.9 us per call measured on the GPU machine's host)
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream_handle(stream) -> int:
    if stream is None:
        return _current_stream_handle()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class StepEvents:
    """Caller-owned HIP events for hc_opts_t.step_events (see include/hc.h):
    timing-enabled torch.cuda.Event objects, whose raw hipEvent_t handles the
    call records.  ``mode`` 0 records one event at every step boundary
    (steps + 1 events); mode 1 has each step's kernels stamp two events with
    their own start and end (2 * steps events)."""

    def __init__(self, events, mode: int = 0):
        self.events = list(events)
        self.mode = int(mode)
        for e in self.events:
            e.record()  # makes torch create the underlying hipEvent_t
        self._arr = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])

    @classmethod
    def for_steps(cls, steps: int, mode: int = 0):
        n = 2 * steps if mode == 1 else steps + 1
        return cls([torch.cuda.Event(enable_timing=True) for _ in range(n)], mode)

    def elapsed_ms(self):
        """Per-step durations in ms: between boundaries (mode 0), or each
        step's own start-to-end stamps (mode 1)."""
        ev = self.events
        if self.mode == 1:
            return [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(len(ev) // 2)]
        return [ev[k].elapsed_time(ev[k + 1]) for k in range(len(ev) - 1)]


def _opts(chunk_fraction: float = 0.0, cu_budget: int = 0, step_events: StepEvents | None = None,
          copy_engine: int = 0):
    if chunk_fraction == 0.0 and cu_budget == 0 and step_events is None and copy_engine == 0:
        return None
    o = hc_opts_t(chunk_fraction, cu_budget, 0, None, int(copy_engine), 0)
    if step_events is not None:
        o.n_step_events = len(step_events.events)
        o.step_events = ctypes.cast(step_events._arr, ctypes.c_void_p)
        o.step_event_mode = step_events.mode
    return ctypes.pointer(o)


def _ptr_array(tensors: Sequence[torch.Tensor], need_elems: int, name: str):
    """The device addresses as a ctypes array, passed where the C call takes
    void *const * (ctypes hands an array to a pointer parameter as the
    address of its first element; an explicit cast cost 2 us per call).
    Returns the array twice: the second reference keeps it alive until the
    call returns."""
    ptrs = []
    for r, t in enumerate(tensors):
        if not t.is_cuda:
            raise ValueError(f"{name}[{r}] is not a device tensor")
        if not t.is_contiguous() or t.numel() < need_elems:
            raise ValueError(f"{name}[{r}] must be contiguous with >= {need_elems} elements")
        ptrs.append(t.data_ptr())
    arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    return arr, arr


def _dptr(t: torch.Tensor | None, need_bytes: int, name: str) -> int | None:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if t.numel() * t.element_size() < need_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {need_bytes}")
    return t.data_ptr()


# ----------------------------------------------------------------------------- ring

def hc_allreduce(sendbufs, recvbufs, count: int | None = None, *, chunk_fraction: float = 0.0,
                 cu_budget: int = 0, step_events: StepEvents | None = None, copy_engine: int = 0,
                 stream=None):
    L = load()
    R = len(sendbufs)
    if count is None:
        count = sendbufs[0].numel()
    if len(recvbufs) != R:
        raise ValueError("sendbufs and recvbufs need one tensor per rank")
    dt = _dtype(sendbufs[0])
    if any(t.dtype != sendbufs[0].dtype for t in list(sendbufs) + list(recvbufs)):
        raise TypeError("all buffers need one dtype")
    sp, _k1 = _ptr_array(sendbufs, count, "sendbufs")
    rp, _k2 = _ptr_array(recvbufs, count, "recvbufs")
    _check(L.hc_allreduce(sp, rp, count, dt, R, _opts(chunk_fraction, cu_budget, step_events, copy_engine),
                          _stream_handle(stream)))


def hc_allreduce_bf16_f32carry(sendbufs, recvbufs, count: int | None = None, ws=None, *,
                               chunk_fraction: float = 0.0, cu_budget: int = 0,
                               step_events: StepEvents | None = None, copy_engine: int = 0, stream=None):
    """bf16 ring allreduce with fp32 partials and one final rounding (see
    include/hc.h); ws: hc_workspace_bytes(HC_OP_ALLREDUCE_F32_CARRY, ...)
    bytes, may be None for one or two ranks."""
    L = load()
    R = len(sendbufs)
    if count is None:
        count = sendbufs[0].numel()
    if len(recvbufs) != R:
        raise ValueError("sendbufs and recvbufs need one tensor per rank")
    if any(t.dtype != torch.bfloat16 for t in list(sendbufs) + list(recvbufs)):
        raise TypeError("the fp32-carry allreduce takes bfloat16 buffers")
    sp, _k1 = _ptr_array(sendbufs, count, "sendbufs")
    rp, _k2 = _ptr_array(recvbufs, count, "recvbufs")
    need = hc_workspace_bytes(HC_OP_ALLREDUCE_F32_CARRY, count, R, HC_BF16)
    wsp = _dptr(ws, need, "ws") if ws is not None else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(L.hc_allreduce_bf16_f32carry(sp, rp, count, R, wsp, ws_bytes,
                                        _opts(chunk_fraction, cu_budget, step_events, copy_engine),
                                        _stream_handle(stream)))


def hc_allreduce_sgd(grads, weights, lr: float, count: int | None = None, *, chunk_fraction: float = 0.0,
                     cu_budget: int = 0, step_events: StepEvents | None = None, copy_engine: int = 0,
                     stream=None):
    """Allreduce of grads fused with weights <- weights - lr * sum (see
    include/hc.h); grads are overwritten with partial sums."""
    L = load()
    R = len(grads)
    if len(weights) != R:
        raise ValueError("one weight buffer per rank")
    if count is None:
        count = grads[0].numel()
    dt = _dtype(grads[0])
    if any(t.dtype != grads[0].dtype for t in list(grads) + list(weights)):
        raise TypeError("all buffers need one dtype")
    gp, _k1 = _ptr_array(grads, count, "grads")
    wp, _k2 = _ptr_array(weights, count, "weights")
    _check(L.hc_allreduce_sgd(gp, wp, count, dt, R, float(lr),
                              _opts(chunk_fraction, cu_budget, step_events, copy_engine), _stream_handle(stream)))


def hc_reduce_scatter(sendbufs, recvbufs, recvcount: int | None = None, ws=None, *,
                      chunk_fraction: float = 0.0, cu_budget: int = 0,
                      step_events: StepEvents | None = None, copy_engine: int = 0, stream=None):
    L = load()
    R = len(sendbufs)
    if recvcount is None:
        recvcount = recvbufs[0].numel()
    dt = _dtype(sendbufs[0])
    if any(t.dtype != sendbufs[0].dtype for t in list(sendbufs) + list(recvbufs)):
        raise TypeError("all buffers need one dtype")
    sp, _k1 = _ptr_array(sendbufs, recvcount * R, "sendbufs")
    rp, _k2 = _ptr_array(recvbufs, recvcount, "recvbufs")
    need = hc_workspace_bytes(HC_OP_REDUCE_SCATTER, recvcount * R, R, dt)
    wsp = _dptr(ws, need, "ws") if ws is not None else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(L.hc_reduce_scatter(sp, rp, recvcount, dt, R, wsp, ws_bytes,
                               _opts(chunk_fraction, cu_budget, step_events, copy_engine), _stream_handle(stream)))


def hc_all_gather(sendbufs, recvbufs, sendcount: int | None = None, *, chunk_fraction: float = 0.0,
                  cu_budget: int = 0, step_events: StepEvents | None = None, copy_engine: int = 0,
                  stream=None):
    L = load()
    R = len(sendbufs)
    if sendcount is None:
        sendcount = sendbufs[0].numel()
    dt = _dtype(sendbufs[0])
    if any(t.dtype != sendbufs[0].dtype for t in list(sendbufs) + list(recvbufs)):
        raise TypeError("all buffers need one dtype")
    sp, _k1 = _ptr_array(sendbufs, sendcount, "sendbufs")
    rp, _k2 = _ptr_array(recvbufs, sendcount * R, "recvbufs")
    _check(L.hc_all_gather(sp, rp, sendcount, dt, R, _opts(chunk_fraction, cu_budget, step_events, copy_engine),
                           _stream_handle(stream)))


def hc_workspace_bytes(op: int, count: int, nranks: int, dtype: int = HC_BF16) -> int:
    return int(load().hc_workspace_bytes(op, count, nranks, dtype))


def hc_chunk_elems(count: int, chunk_fraction: float = 0.01, align: int = 1024) -> int:
    return int(load().hc_chunk_elems(count, chunk_fraction, align))


def hc_ring_tasks(nranks: int, count: int, chunk: int):
    L = load()
    n = int(L.hc_ring_tasks(nranks, count, chunk, None, 0))
    buf = (hc_task_t * max(n, 1))()
    L.hc_ring_tasks(nranks, count, chunk, buf, n)
    return [(t.src, t.dst, t.step, t.chunk, t.op, t.slice, t.off, t.len) for t in buf[:n]]


# ----------------------------------------------------------------------------- codec

def hc_compress_bound_bf16(n: int) -> int:
    return int(load().hc_compress_bound_bf16(n))


def hc_compress_bf16(d_in: torch.Tensor, n: int, d_out: torch.Tensor, d_out_bytes: torch.Tensor,
                     ws: torch.Tensor, *, stream=None):
    L = load()
    if d_in.element_size() != 2:
        raise TypeError("input must hold 16-bit words")
    inp = _dptr(d_in, 2 * n, "d_in") if n else (d_in.data_ptr() if d_in.numel() else None)
    out_cap = d_out.numel() * d_out.element_size()
    outp = _dptr(d_out, 1, "d_out")
    ob = _dptr(d_out_bytes, 8, "d_out_bytes")
    wsp = _dptr(ws, 1, "ws")
    _check(L.hc_compress_bf16(inp, n, outp, out_cap, ob, wsp, ws.numel() * ws.element_size(),
                              _stream_handle(stream)))


def hc_compress_bf16_noalloc(d_in: torch.Tensor, n: int, d_out: torch.Tensor, d_out_bytes: torch.Tensor, *,
                             stream=None):
    """hc_compress_bf16 with the library's static scratch instead of a
    workspace (allocates nothing; n <= 2^31)."""
    L = load()
    if d_in.element_size() != 2:
        raise TypeError("input must hold 16-bit words")
    inp = _dptr(d_in, 2 * n, "d_in") if n else (d_in.data_ptr() if d_in.numel() else None)
    out_cap = d_out.numel() * d_out.element_size()
    outp = _dptr(d_out, 1, "d_out")
    ob = _dptr(d_out_bytes, 8, "d_out_bytes")
    _check(L.hc_compress_bf16_noalloc(inp, n, outp, out_cap, ob, _stream_handle(stream)))


def hc_compress_bf16_scoped(d_in: torch.Tensor, n: int, d_out: torch.Tensor, d_out_bytes: torch.Tensor,
                            table_blocks: int, ws: torch.Tensor, *, stream=None):
    """hc_compress_bf16 with one code table per table_blocks full blocks
    (0: one table for the whole stream)."""
    L = load()
    if d_in.element_size() != 2:
        raise TypeError("input must hold 16-bit words")
    if table_blocks < 0:
        raise ValueError("table_blocks must be >= 0")
    inp = _dptr(d_in, 2 * n, "d_in") if n else (d_in.data_ptr() if d_in.numel() else None)
    out_cap = d_out.numel() * d_out.element_size()
    outp = _dptr(d_out, 1, "d_out")
    ob = _dptr(d_out_bytes, 8, "d_out_bytes")
    wsp = _dptr(ws, 1, "ws")
    _check(L.hc_compress_bf16_scoped(inp, n, outp, out_cap, ob, table_blocks, wsp,
                                     ws.numel() * ws.element_size(), _stream_handle(stream)))


def hc_decompress_bf16(d_in: torch.Tensor, in_bytes: int, d_out: torch.Tensor, n: int,
                       d_status: torch.Tensor, *, stream=None):
    L = load()
    inp = _dptr(d_in, in_bytes, "d_in")
    outp = _dptr(d_out, 2 * n, "d_out") if n else None
    st = _dptr(d_status, 4, "d_status")
    _check(L.hc_decompress_bf16(inp, in_bytes, outp, n, st, _stream_handle(stream)))


def hc_compress_bf16_staged(d_in: torch.Tensor, n: int, d_out: torch.Tensor, d_out_bytes: torch.Tensor,
                            ws: torch.Tensor, *, stream=None):
    """hc_compress_bf16 in three global rounds (slots, prefix, coalescing copy)."""
    L = load()
    if d_in.element_size() != 2:
        raise TypeError("input must hold 16-bit words")
    inp = _dptr(d_in, 2 * n, "d_in") if n else (d_in.data_ptr() if d_in.numel() else None)
    out_cap = d_out.numel() * d_out.element_size()
    outp = _dptr(d_out, 1, "d_out")
    ob = _dptr(d_out_bytes, 8, "d_out_bytes")
    wsp = _dptr(ws, 1, "ws")
    _check(L.hc_compress_bf16_staged(inp, n, outp, out_cap, ob, wsp, ws.numel() * ws.element_size(),
                                     _stream_handle(stream)))


def hc_compress_bf16_entropy(d_in: torch.Tensor, n: int, d_out: torch.Tensor, d_out_bytes: torch.Tensor,
                             ws: torch.Tensor, *, stream=None):
    """HCE1 stream: per-block canonical Huffman codes for the exponent."""
    L = load()
    if d_in.element_size() != 2:
        raise TypeError("input must hold 16-bit words")
    inp = _dptr(d_in, 2 * n, "d_in") if n else (d_in.data_ptr() if d_in.numel() else None)
    out_cap = d_out.numel() * d_out.element_size()
    outp = _dptr(d_out, 1, "d_out")
    ob = _dptr(d_out_bytes, 8, "d_out_bytes")
    wsp = _dptr(ws, 1, "ws")
    _check(L.hc_compress_bf16_entropy(inp, n, outp, out_cap, ob, wsp, ws.numel() * ws.element_size(),
                                      _stream_handle(stream)))


def hc_decompress_bf16_entropy(d_in: torch.Tensor, in_bytes: int, d_out: torch.Tensor, n: int,
                               d_status: torch.Tensor, *, stream=None):
    L = load()
    inp = _dptr(d_in, in_bytes, "d_in")
    outp = _dptr(d_out, 2 * n, "d_out") if n else None
    st = _dptr(d_status, 4, "d_status")
    _check(L.hc_decompress_bf16_entropy(inp, in_bytes, outp, n, st, _stream_handle(stream)))


def hc_compressed_allreduce(sendbufs, recvbufs, count: int | None, ws: torch.Tensor,
                            d_wire_bytes: torch.Tensor | None = None, *, chunk_fraction: float = 0.0,
                            step_events: StepEvents | None = None, stream=None):
    L = load()
    R = len(sendbufs)
    if count is None:
        count = sendbufs[0].numel()
    if any(t.dtype != torch.bfloat16 for t in list(sendbufs) + list(recvbufs)):
        raise TypeError("compressed allreduce is bf16 only")
    sp, _k1 = _ptr_array(sendbufs, count, "sendbufs")
    rp, _k2 = _ptr_array(recvbufs, count, "recvbufs")
    wsp = _dptr(ws, 1, "ws")
    wb = _dptr(d_wire_bytes, 8, "d_wire_bytes") if d_wire_bytes is not None else None
    _check(L.hc_compressed_allreduce(sp, rp, count, R, wsp, ws.numel() * ws.element_size(), wb,
                                     _opts(chunk_fraction, 0, step_events), _stream_handle(stream)))


# ----------------------------------------------------------------------------- streams

def hc_stream_create_cu_budget(k: int) -> int:
    """Returns the raw hipStream_t handle; wrap it with torch.cuda.ExternalStream."""
    L = load()
    s = ctypes.c_void_p(0)
    _check(L.hc_stream_create_cu_budget(k, ctypes.byref(s)))
    return int(s.value)


def hc_stream_create_cu_range(first: int, k: int) -> int:
    """A stream on CU mask bits [first, first + k); returns the raw handle."""
    L = load()
    s = ctypes.c_void_p(0)
    _check(L.hc_stream_create_cu_range(first, k, ctypes.byref(s)))
    return int(s.value)


def hc_stream_destroy(handle: int):
    _check(load().hc_stream_destroy(handle))


def hc_cu_census(n_workgroups: int, hold_us: int = 50, *, stream=None):
    """Where n_workgroups one-wave workgroups run on `stream`: a (n, 2)
    int64 tensor of (XCC_ID & 15, HW_ID bits 8..15) per workgroup, after the
    launch completes (synchronises the stream)."""
    L = load()
    ids = torch.zeros(2 * n_workgroups, dtype=torch.int32, device="cuda")
    _check(L.hc_cu_census(ids.data_ptr(), n_workgroups, hold_us, _stream_handle(stream)))
    if stream is None:
        torch.cuda.current_stream().synchronize()
    elif isinstance(stream, int):
        torch.cuda.synchronize()
    else:
        stream.synchronize()
    h = ids.view(-1, 2).cpu().to(torch.int64)
    return torch.stack([h[:, 1] & 15, (h[:, 0] >> 8) & 0xFF], dim=1)


def hc_step_count(op: int, nranks: int) -> int:
    return int(load().hc_step_count(op, nranks))


def hc_copy_engine_available() -> bool:
    """True when this process's HIP runtime puts copy_engine copies on the DMA
    engines (else copy_engine=1 raises HcError with HC_ERR_UNSUPPORTED)."""
    return bool(load().hc_copy_engine_available())


def hc_version() -> str:
    return load().hc_version().decode()
