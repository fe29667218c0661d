"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no arithmetic of the method (no reduction, no codec, no
bf16 rounding rule of its own): it draws numbers with numpy and converts fp32
to bf16 with PyTorch's CPU conversion (round to nearest even), and nothing
else.  The same host bytes feed both the GPU path and the oracle.

Workloads (tensor shapes of gradients, weights and activations as the pages
describe them; the pages' nccl-tests sweeps span 2 MB to 1 GB per message):

* ``ring_f32``   -- R=4 ranks x 2^20 fp32, N(0, 1)
* ``ring_bf16``  -- R=8 ranks x 2^26 bf16, N(0, 1e-3), 1% of entries zero
* ``codec``      -- 2^28 bf16 each: weights N(0, 0.02); activations a 50/50
  per-element mixture of N(0, 1) and Laplace(0, 4); gradients N(0, 1e-4)
* ``compressed`` -- R=8 ranks x 2^25 bf16, N(0, 1e-3)
* ``contention`` -- R=8 ranks x 2^28 bf16, N(0, 1e-3)
* ``bucket``     -- a flattened gradient bucket of many layers: layer sizes
  log-uniform in [2^12, 2^22) elements (so layer edges fall inside codec
  blocks), layer l drawn N(0, s_l) with s_l log-uniform in [1e-5, 1e-1]

N(mu, s) names the standard deviation s.  Seeds are
``SeedSequence([20261202, workload_id, index])``.  Two generators draw from
that seed: numpy's default generator on the host (``device="cpu"``, used for
test-sized inputs) and torch's Philox generator on the GPU (``device="cuda"``,
for the full-size workloads, whose billions of draws the host generator would
take minutes over); the GPU path returns a device tensor whose host copy is
what the oracle sees.
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 20261202

WORKLOAD_IDS = {"ring_f32": 1, "ring_bf16": 2, "codec": 3, "compressed": 4, "contention": 5,
                "fused_sgd": 6, "bucket": 7, "test": 99}


def rng_for(workload: str | int, index: int) -> np.random.Generator:
    wid = WORKLOAD_IDS[workload] if isinstance(workload, str) else int(workload)
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, wid, int(index)]))


def seed64(workload: str | int, index: int) -> int:
    wid = WORKLOAD_IDS[workload] if isinstance(workload, str) else int(workload)
    return int(np.random.SeedSequence([ROOT_SEED, wid, int(index)]).generate_state(1, np.uint64)[0] >> 1)


def _cuda_gen(workload, index):
    import torch

    g = torch.Generator(device="cuda")
    g.manual_seed(seed64(workload, index))
    return g


def normal_bf16_cuda(workload, index: int, n: int, sigma: float, zero_frac: float = 0.0):
    """Device bf16 tensor: N(0, sigma) rounded to bf16 (nearest even), with an
    independent Bernoulli(zero_frac) mask of exact zeros."""
    import torch

    g = _cuda_gen(workload, index)
    x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
    x.mul_(sigma)
    if zero_frac > 0.0:
        u = torch.rand(n, generator=g, device="cuda", dtype=torch.float32)
        x.masked_fill_(u < zero_frac, 0.0)
        del u
    return x.to(torch.bfloat16)


def bucket_layers(workload, index: int, n: int):
    """Layer plan of a gradient bucket of n elements: (sizes, sigmas), drawn
    on the host from the seed; the last layer is cut to fill n exactly."""
    return _bucket_plan(rng_for(workload, index), n)


def _bucket_plan(g: np.random.Generator, n: int):
    sizes, sigmas, total = [], [], 0
    while total < n:
        size = int(2.0 ** g.uniform(12.0, 22.0))
        size = min(size, n - total)
        sizes.append(size)
        sigmas.append(float(10.0 ** g.uniform(-5.0, -1.0)))
        total += size
    return sizes, sigmas


def bucket_bf16_cuda(workload, index: int, n: int):
    """Device bf16 tensor: a gradient bucket (see bucket_layers)."""
    import torch

    sizes, sigmas = bucket_layers(workload, index, n)
    g = _cuda_gen(workload, index)
    x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
    scale = torch.repeat_interleave(torch.tensor(sigmas, dtype=torch.float32),
                                    torch.tensor(sizes, dtype=torch.int64)).to("cuda")
    x.mul_(scale)
    del scale
    return x.to(torch.bfloat16)


def activation_bf16_cuda(workload, index: int, n: int):
    """Device bf16 tensor: per-element 50/50 mixture of N(0, 1) and Laplace(0, 4)
    (Laplace drawn by the inverse CDF of a uniform on (-1/2, 1/2))."""
    import torch

    g = _cuda_gen(workload, index)
    pick = torch.rand(n, generator=g, device="cuda") < 0.5
    x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
    u = torch.rand(n, generator=g, device="cuda", dtype=torch.float64) - 0.5
    lap = (-4.0 * torch.sign(u) * torch.log1p(-2.0 * u.abs())).to(torch.float32)
    x = torch.where(pick, lap, x)
    return x.to(torch.bfloat16)


def normal_f32_cuda(workload, index: int, n: int, sigma: float = 1.0):
    import torch

    g = _cuda_gen(workload, index)
    x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x


def ring_inputs_cuda(workload: str, R: int, n: int):
    """Per-rank device tensors of a ring workload."""
    if workload == "ring_f32":
        return [normal_f32_cuda(workload, r, n, 1.0) for r in range(R)]
    if workload == "ring_bf16":
        return [normal_bf16_cuda(workload, r, n, 1e-3, zero_frac=0.01) for r in range(R)]
    if workload in ("compressed", "contention"):
        return [normal_bf16_cuda(workload, r, n, 1e-3) for r in range(R)]
    raise KeyError(workload)


def codec_inputs_cuda(n: int):
    return {
        "weights": normal_bf16_cuda("codec", 0, n, 0.02),
        "activations": activation_bf16_cuda("codec", 1, n),
        "gradients": normal_bf16_cuda("codec", 2, n, 1e-4),
    }


def host_bits(t) -> np.ndarray:
    """Device tensor -> host bit patterns (uint16 for bf16, float32 as is)."""
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) by PyTorch's CPU conversion (nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_f32(workload, index: int, n: int, sigma: float = 1.0) -> np.ndarray:
    g = rng_for(workload, index)
    x = g.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def normal_bf16(workload, index: int, n: int, sigma: float, zero_frac: float = 0.0) -> np.ndarray:
    g = rng_for(workload, index)
    x = g.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    if zero_frac > 0.0:
        x[g.random(n, dtype=np.float32) < zero_frac] = 0.0
    return f32_to_bf16_bits(x)


def activation_bf16(workload, index: int, n: int) -> np.ndarray:
    """Per-element 50/50 mixture of N(0, 1) and Laplace(0, scale 4)."""
    g = rng_for(workload, index)
    pick = g.random(n, dtype=np.float32) < 0.5
    x = g.standard_normal(n, dtype=np.float32)
    lap = g.laplace(0.0, 4.0, n).astype(np.float32)
    x[pick] = lap[pick]
    return f32_to_bf16_bits(x)


def bucket_bf16(workload, index: int, n: int) -> np.ndarray:
    """Host bf16 bits of a gradient bucket (see bucket_layers)."""
    g = rng_for(workload, index)
    sizes, sigmas = _bucket_plan(g, n)
    x = g.standard_normal(n, dtype=np.float32)
    x *= np.repeat(np.array(sigmas, dtype=np.float32), sizes)
    return f32_to_bf16_bits(x)


def ring_inputs(workload: str, R: int, n: int):
    """Per-rank inputs of a ring workload (list of R arrays)."""
    if workload == "ring_f32":
        return [normal_f32(workload, r, n, 1.0) for r in range(R)]
    if workload == "ring_bf16":
        return [normal_bf16(workload, r, n, 1e-3, zero_frac=0.01) for r in range(R)]
    if workload in ("compressed", "contention"):
        return [normal_bf16(workload, r, n, 1e-3) for r in range(R)]
    raise KeyError(workload)


def codec_inputs(n: int):
    """The three codec tensors: weights, activations, gradients (bf16 bits)."""
    return {
        "weights": normal_bf16("codec", 0, n, 0.02),
        "activations": activation_bf16("codec", 1, n),
        "gradients": normal_bf16("codec", 2, n, 1e-4),
    }
