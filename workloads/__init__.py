"""Seeded synthetic inputs for the n-rank reduction path.

This module is shared by the tests, the smoke check and the benchmark: it
creates rank buffers and nothing else.  It holds none of the reduction's
arithmetic and imports neither the oracle nor the product library.

Every buffer is drawn from numpy's PCG64 via ``default_rng([seed, stream,
rank])`` (one independent substream per rank), or, for buffers too large to
draw on the host in reasonable time, from torch's device Philox generator
seeded with the same triple.  Sizes use binary units (KB = 2^10 bytes, MB =
2^20, GB = 2^30).

The five workloads (value distributions and shapes of the pages' workloads;
the pages measure with nccl-tests sweeps and real gradient buckets, which
these stand in for):

* ``c1`` -- all-reduce, n = 4, fp32, 1024 elements per rank, integers uniform
  in [-8, 8] stored as fp32 (sums are exact), seed 0.
* ``c2`` -- all-reduce, n = 8, fp32, 64 Mi elements (256 MB) per rank,
  N(0, sigma = 1e-3), seed 1.
* ``c3`` -- FSDP-style reduce-scatter (avg) of 128 Mi bf16 per rank
  (N(0, 1e-2), seed 2 stream 0) and all-gather of 16 Mi bf16 per rank
  (uniform [-1, 1], seed 2 stream 1).
* ``c4`` -- message-size sweep, n = 16, int32 uniform in [-2^20, 2^20],
  per-rank sizes 1 KB .. 1 GB in powers of 4 (seed 3, stream log2(bytes)).
* ``c5`` -- bucketed gradient all-reduce, n = 72, fp32, 256 tensors with byte
  sizes 16*floor(exp(U(ln 2^12, ln 2^24))/16) (seed 4, stream 0), packed in
  reverse order into 25 MB buckets; values N(0, 1e-3) (seed 4, stream 1) with
  an independent 1 % Bernoulli mask (stream 2) scaling entries by 100.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KB = 1 << 10
MB = 1 << 20
GB = 1 << 30

ELEM_SIZE = {"f32": 4, "bf16": 2, "f16": 2, "i32": 4}


def rng(seed: int, stream: int, rank: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream, rank])


# ---------------------------------------------------------------------------
# host generators (numpy); bf16 arrays are returned as uint16 bit patterns
# ---------------------------------------------------------------------------

def _f32_to_bf16_bits_host(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (torch's CPU conversion, round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def ints(seed, stream, rank, count, lo, hi, dtype="f32"):
    """Integers uniform in [lo, hi] (inclusive), stored as ``dtype``."""
    v = rng(seed, stream, rank).integers(lo, hi, size=count, endpoint=True, dtype=np.int64)
    if dtype == "i32":
        return v.astype(np.int32)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    return _f32_to_bf16_bits_host(v.astype(np.float32))


def normal(seed, stream, rank, count, sigma, dtype="f32"):
    """N(0, sigma) samples (sigma is the standard deviation), stored as ``dtype``."""
    v = rng(seed, stream, rank).standard_normal(count, dtype=np.float32) * np.float32(sigma)
    if dtype == "f32":
        return v
    if dtype == "f16":
        return v.astype(np.float16)
    return _f32_to_bf16_bits_host(v)


def uniform(seed, stream, rank, count, lo, hi, dtype="f32"):
    v = rng(seed, stream, rank).uniform(lo, hi, size=count).astype(np.float32)
    if dtype == "f32":
        return v
    if dtype == "f16":
        return v.astype(np.float16)
    return _f32_to_bf16_bits_host(v)


# Scales of the ``extremes`` test data per float type: a factor that puts
# N(0,1) samples among the type's subnormals, and a large magnitude whose sums
# over a few ranks overflow to infinity.
_TINY = {"f32": 2.0 ** -140, "bf16": 2.0 ** -130, "f16": 2.0 ** -20}
_HUGE = {"f32": 2.0 ** 127, "bf16": 2.0 ** 127, "f16": 2.0 ** 14}


def extremes(seed, stream, rank, count, dtype):
    """Float test data by element position (the same class on every rank):
    i % 4 == 0: N(0,1); 1: subnormal-range values; 2: large positive values
    (sums and products overflow to +inf, never inf - inf); 3: N(0,1) on even
    ranks, subnormal-range on odd ones."""
    g = rng(seed, stream, rank)
    z = g.standard_normal(count)
    big = g.uniform(0.5, 1.0, size=count)
    cls = np.arange(count) % 4
    tiny = _TINY[dtype]
    v = np.where(cls == 0, z, np.where(cls == 1, z * tiny, np.where(cls == 2, big * _HUGE[dtype],
                                                                     z * (1.0 if rank % 2 == 0 else tiny))))
    if dtype == "f16":
        return v.astype(np.float16)
    v32 = v.astype(np.float32)
    return v32 if dtype == "f32" else _f32_to_bf16_bits_host(v32)


def random_values(seed, stream, rank, count, dtype, kind="normal"):
    """Generic test data: ``normal`` (N(0,1)), ``ints`` (small integers), ``pos``
    (uniform [0.5, 2]) or ``extremes`` (float types: subnormals and overflow)."""
    if kind == "extremes":
        return extremes(seed, stream, rank, count, dtype)
    if kind == "ints":
        lo, hi = (-(1 << 20), 1 << 20) if dtype == "i32" else (-8, 8)
        return ints(seed, stream, rank, count, lo, hi, dtype)
    if kind == "pos":
        if dtype == "i32":
            return ints(seed, stream, rank, count, -3, 3, dtype)
        return uniform(seed, stream, rank, count, 0.5, 2.0, dtype)
    if dtype == "i32":
        return ints(seed, stream, rank, count, -(1 << 30), 1 << 30, dtype)
    return normal(seed, stream, rank, count, 1.0, dtype)


# ---------------------------------------------------------------------------
# device generators (torch Philox), for buffers of hundreds of MB per rank
# ---------------------------------------------------------------------------

def _torch_gen(seed, stream, rank, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream) * 1_000_033 + rank)
    return g


def device_normal(seed, stream, rank, count, sigma, dtype, device="cuda"):
    import torch
    g = _torch_gen(seed, stream, rank, device)
    t = torch.randn(count, generator=g, device=device, dtype=torch.float32)
    t.mul_(sigma)
    return _device_cast(t, dtype)


def device_uniform(seed, stream, rank, count, lo, hi, dtype, device="cuda"):
    import torch
    g = _torch_gen(seed, stream, rank, device)
    t = torch.empty(count, device=device, dtype=torch.float32).uniform_(lo, hi, generator=g)
    return _device_cast(t, dtype)


def device_ints(seed, stream, rank, count, lo, hi, dtype, device="cuda"):
    import torch
    g = _torch_gen(seed, stream, rank, device)
    t = torch.randint(lo, hi + 1, (count,), generator=g, device=device, dtype=torch.int32)
    if dtype == "i32":
        return t
    return _device_cast(t.to(torch.float32), dtype)


def device_spiky_normal(seed, rank, count, sigma, frac, scale, device="cuda"):
    """N(0, sigma) fp32 with an independent Bernoulli(frac) mask scaled by ``scale``."""
    import torch
    t = device_normal(seed, 1, rank, count, sigma, "f32", device)
    g = _torch_gen(seed, 2, rank, device)
    m = torch.rand(count, generator=g, device=device) < frac
    t[m] *= scale
    return t


def _device_cast(t, dtype):
    import torch
    return t.to({"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
                 "i32": torch.int32}[dtype])


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    n: int
    dtype: str
    count: int                      # elements per rank (all-reduce) or per-rank input (reduce-scatter)
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def bytes_per_rank(self) -> int:
        return self.count * ELEM_SIZE[self.dtype]


C1 = Workload("c1_ar_n4_f32_1024", 4, "f32", 1024, "integers in [-8, 8] as fp32, seed 0")
C2 = Workload("c2_ar_n8_f32_256MB", 8, "f32", 64 * MB, "N(0, 1e-3), seed 1")
C3_RS = Workload("c3_rs_n8_bf16_256MB", 8, "bf16", 128 * MB, "N(0, 1e-2) as bf16, seed 2 stream 0")
C3_AG = Workload("c3_ag_n8_bf16_32MB", 8, "bf16", 16 * MB, "uniform [-1, 1] as bf16, seed 2 stream 1")
C4_SIZES = [KB << (2 * k) for k in range(11)]          # 1 KB .. 1 GB per rank, powers of 4
C4_N = 16
C5_N = 72
C5_BUCKET_BYTES = 25 * MB


def c1_inputs():
    return [ints(0, 0, r, C1.count, -8, 8, "f32") for r in range(C1.n)]


def c4_host_inputs(size_bytes: int, n: int = C4_N):
    stream = int(math.log2(size_bytes))
    return [ints(3, stream, r, size_bytes // 4, -(1 << 20), 1 << 20, "i32") for r in range(n)]


def c5_tensor_sizes(num: int = 256) -> list[int]:
    """Byte sizes of the 256 gradient tensors, log-uniform in [4 KB, 16 MB], 16-byte multiples."""
    u = rng(4, 0, 0).uniform(math.log(4 * KB), math.log(16 * MB), size=num)
    return [16 * int(math.floor(math.exp(x) / 16)) for x in u]


def c5_buckets(bucket_bytes: int = C5_BUCKET_BYTES):
    """Pack the tensors in reverse order (last layer's gradients are ready first)
    greedily into buckets of at most ``bucket_bytes``; a tensor larger than a
    bucket gets a bucket of its own.  Returns [(byte_offset, byte_size)] of
    each bucket within the flat per-rank gradient buffer, and the total size."""
    sizes = c5_tensor_sizes()[::-1]
    buckets, cur_off, cur = [], 0, 0
    for s in sizes:
        if cur and cur + s > bucket_bytes:
            buckets.append((cur_off, cur))
            cur_off += cur
            cur = 0
        cur += s
    if cur:
        buckets.append((cur_off, cur))
        cur_off += cur
    return buckets, cur_off
