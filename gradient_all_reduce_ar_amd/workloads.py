"""Seeded synthetic inputs for the all-reduce workloads.

This module only draws numbers: it holds none of the all-reduce arithmetic, so
both the GPU library's tests and the CPU oracle can take their inputs from it.

Workloads (shapes from "Chapter 7. Data-center networks", section 7.2.1,
which uses the fp32 [12288, 4096] FFN gate-projection gradient of Qwen3-8B,
192 MiB per rank; values are synthetic, no gradients or weights are used):

  uniform  : x_r ~ U[-1, 1) fp32 from default_rng([seed, r])
  normal   : x_r ~ N(0, sigma) fp32 from default_rng([seed, r]); for bf16 the
             fp32 draw is rounded to bf16 by torch's conversion
  bucketed : 300 tensors whose byte sizes are lognormal (median 256 KiB),
             values N(0, 1e-3) per (rank, tensor), bf16
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GATE_PROJ_ELEMS = 12288 * 4096  # 50,331,648 fp32 elements = 192 MiB
BF16_192MIB_ELEMS = 2 * GATE_PROJ_ELEMS  # 100,663,296 bf16 elements = 192 MiB


def _to_bf16_bits(x):
    """fp32 numpy array -> uint16 array of bf16 bits (torch's conversion)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def uniform_rank(r, count, seed=0):
    rng = np.random.default_rng([seed, r])
    return (rng.random(count, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)).astype(np.float32)


def normal_rank(r, count, seed=0, sigma=1e-3, dtype="fp32"):
    rng = np.random.default_rng([seed, r])
    x = rng.standard_normal(count, dtype=np.float32) * np.float32(sigma)
    return x if dtype == "fp32" else _to_bf16_bits(x)


def _per_rank(fn, nranks):
    # each rank draws from its own generator, so threads give the same numbers
    if nranks <= 1:
        return [fn(r) for r in range(nranks)]
    with ThreadPoolExecutor(min(8, nranks)) as ex:
        return list(ex.map(fn, range(nranks)))


def uniform_inputs(nranks, count, seed=0, dtype="fp32"):
    xs = _per_rank(lambda r: uniform_rank(r, count, seed), nranks)
    return xs if dtype == "fp32" else [_to_bf16_bits(x) for x in xs]


def normal_inputs(nranks, count, seed=0, sigma=1e-3, dtype="fp32"):
    return _per_rank(lambda r: normal_rank(r, count, seed, sigma, dtype), nranks)


def integer_inputs(nranks, count, seed=0, lo=-8, hi=8, dtype="fp32"):
    """Small integers (exactly representable partial sums for small N)."""
    xs = []
    for r in range(nranks):
        rng = np.random.default_rng([seed, r, 17])
        xs.append(rng.integers(lo, hi, count).astype(np.float32))
    return xs if dtype == "fp32" else [_to_bf16_bits(x) for x in xs]


def bucketed_tensor_sizes(ntensors=300, seed=7, median_bytes=262144, sigma=2.0,
                          min_bytes=512, max_bytes=64 << 20, elem_bytes=2):
    """Element counts of the gradient tensors of one rank.

    Byte sizes are lognormal(ln median, sigma), clipped to [min, max], rounded
    to whole elements; the largest tensor is then set to exactly max_bytes.
    """
    rng = np.random.default_rng(seed)
    b = rng.lognormal(np.log(median_bytes), sigma, ntensors)
    b = np.clip(b, min_bytes, max_bytes)
    counts = np.maximum(1, np.round(b / elem_bytes)).astype(np.int64)
    counts[int(np.argmax(counts))] = max_bytes // elem_bytes
    return counts


def bucketed_tensor_values(r, t, count, seed=0, sigma=1e-3, dtype="bf16"):
    rng = np.random.default_rng([seed, r, t])
    x = rng.standard_normal(int(count), dtype=np.float32) * np.float32(sigma)
    return x if dtype == "fp32" else _to_bf16_bits(x)


def bucketed_arenas(nranks, sizes, offsets, arena_count, seed=0, sigma=1e-3, dtype="bf16"):
    """Per-rank arenas with tensor t of rank r at offsets[t]; gaps are zero."""
    def fill(r):
        a = np.zeros(arena_count, np.float32 if dtype == "fp32" else np.uint16)
        for t, c in enumerate(sizes):
            a[offsets[t]:offsets[t] + int(c)] = bucketed_tensor_values(r, t, c, seed, sigma, dtype)
        return a
    return _per_rank(fill, nranks)


def device_rank(r, count, seed=0, sigma=1e-3, dtype="fp32", heavy=False, device="cuda:0"):
    """Rank r's input drawn on the device (for buffers too large to stage
    through host memory): x ~ N(0, sigma) fp32 from torch's generator seeded
    with (seed, r); heavy=True multiplies each value by exp(N(0, 1)) so that
    magnitudes vary over several decades.  bf16 is torch's conversion of the
    fp32 draw, returned as int16 storage."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(r))
    x = torch.randn(int(count), generator=g, device=device, dtype=torch.float32)
    x.mul_(sigma)
    if heavy:
        y = torch.randn(int(count), generator=g, device=device, dtype=torch.float32)
        x.mul_(y.exp_())
        del y
    if dtype == "fp32":
        return x
    return x.to(torch.bfloat16).view(torch.int16)
