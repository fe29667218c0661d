"""Helpers for the GPU tests: numpy bit patterns <-> torch device tensors."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev(x: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor; float32 -> float32 tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(dev())
    if x.dtype == np.float32:
        return torch.from_numpy(x.copy()).to(dev())
    raise TypeError(x.dtype)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy bit patterns (uint16 for bf16, uint32 for fp32, uint8 bytes)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    raise TypeError(t.dtype)


def bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    d = np.nonzero(a != b)[0]
    if d.size == 0:
        return "equal"
    i = int(d[0])
    return f"{d.size} mismatches, first at {i}: got 0x{int(a[i]):x} want 0x{int(b[i]):x}"


def fold_chunked(xs, lo: int = 0, hi: int = -1, chunk: int = 1 << 22, threads: int = 8) -> np.ndarray:
    """The oracle's allreduce fold of the whole index range [lo, hi) (default:
    every index), evaluated by the oracle's fold-at-indices in chunks so that
    buffers too large for the whole fold's R outputs can be compared element
    by element.  The chunks run on a few host threads (the oracle call holds
    no Python lock); each call is the plain single-threaded oracle."""
    import concurrent.futures as cf

    import oracle

    n = xs[0].size
    hi = n if hi < 0 else hi
    out = np.empty(hi - lo, dtype=xs[0].dtype)

    def one(a):
        b = min(hi, a + chunk)
        out[a - lo:b - lo] = oracle.allreduce_fold_at(xs, np.arange(a, b, dtype=np.uint64))

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(lo, hi, chunk)))
    return out


def copy_engine_or_unsupported(call):
    """Runs call() (a library call with copy_engine=1).  When this process's
    HIP runtime would not put the copies on the DMA engines, the call must
    refuse with HC_ERR_UNSUPPORTED before enqueueing anything; returns True
    when the call ran."""
    import pytest

    from collective_communication_amd import binding as hc

    if hc.hc_copy_engine_available():
        call()
        return True
    with pytest.raises(hc.HcError) as e:
        call()
    assert e.value.status == hc.HC_ERR_UNSUPPORTED
    assert "DMA engines" in str(e.value)
    return False
