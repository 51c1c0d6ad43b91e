"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage type;
it holds none of the GEMM arithmetic.  Values are drawn in float64 with
numpy's PCG64, converted to float32, then rounded once to the storage dtype
with round-to-nearest-even:

* fp32: stored as is (``uint32`` bit patterns),
* fp16: numpy's float32 -> float16 conversion (IEEE RNE),
* bf16: RNE on the top 16 bits of the float32 pattern.

Every generator returns raw bit patterns (``uint32`` for fp32, ``uint16`` for
fp16/bf16) so the GPU and the oracle read identical bits.
"""
import os
import random
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Values are drawn in fixed chunks of this many elements, chunk i from its own
# PCG64 stream seeded with (seed, i), so they do not depend on the thread count.
CHUNK = 1 << 22


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n, fn):
    """Run fn(i, lo, hi) over the fixed chunks of [0, n) on a thread pool."""
    spans = [(i, lo, min(lo + CHUNK, n)) for i, lo in enumerate(range(0, n, CHUNK))]
    if len(spans) <= 1:
        for sp in spans:
            fn(*sp)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda sp: fn(*sp), spans))

DTYPE_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2}


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    shape = x.shape
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)

    def one(_, lo, hi):
        uc = u[lo:hi]
        nan = np.isnan(uc.view(np.float32))
        t = uc >> 16
        t &= 1
        t += 0x7FFF
        if nan.any():
            t += np.where(nan, np.uint32(0), uc)
        else:
            t += uc  # never wraps: non-NaN patterns are at most 0xff800000
        t >>= 16
        o = t.astype(np.uint16)
        if nan.any():
            o[nan] = ((uc[nan] >> 16) | 0x40).astype(np.uint16)
        out[lo:hi] = o

    _chunked(u.size, one)
    return out.reshape(shape)


def to_bits(x32, dtype):
    """float32 array -> storage bit patterns of ``dtype``."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f32":
        return x32.view(np.uint32).copy()
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "i8":
        # int8 operands are drawn as integers (distributions 'int8', 'int4')
        if not (np.all(x32 == np.round(x32)) and x32.min(initial=0) >= -128
                and x32.max(initial=0) <= 127):
            raise ValueError("i8 operands need integer values in [-128, 127]")
        return x32.astype(np.int8)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(shape, dist, seed, scale=1.0):
    """float32 samples: 'normal' = N(0,1), 'uniform' = U[-1,1), 'int4' = integers in [-4,4],
    'int8' = integers in [-128, 127]."""
    if dist not in ("normal", "uniform", "int4", "int8"):
        raise ValueError(f"unknown distribution {dist!r}")
    x = np.empty(shape, dtype=np.float32)
    flat = x.reshape(-1)

    def one(i, lo, hi):
        rng = np.random.Generator(np.random.PCG64([seed, i]))
        part = flat[lo:hi]
        if dist == "normal":
            rng.standard_normal(out=part, dtype=np.float32)
        elif dist == "uniform":
            rng.random(out=part, dtype=np.float32)
            part *= np.float32(2.0)
            part -= np.float32(1.0)
        elif dist == "int4":
            part[:] = rng.integers(-4, 5, size=hi - lo)
        else:
            part[:] = rng.integers(-128, 128, size=hi - lo)
        if scale != 1.0:
            part *= np.float32(scale)

    _chunked(flat.size, one)
    return x


def operands(M, N, K, dtype, dist, seed, scale=1.0):
    """(A bits M x K, B bits K x N) with A drawn from ``seed`` and B from ``seed + 1``."""
    a = to_bits(draw((M, K), dist, seed, scale), dtype)
    b = to_bits(draw((K, N), dist, seed + 1, scale), dtype)
    return a, b


def sample_positions(M, N, n, seed, tails=False):
    """(rows, cols) int64 arrays: ``n`` seeded uniform output positions.

    With ``tails`` the last two rows, the last two columns and the four
    corners are appended in full (the ragged edges of a tiled output).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = rng.integers(0, M, size=n, dtype=np.int64)
    cols = rng.integers(0, N, size=n, dtype=np.int64)
    if tails:
        r_extra, c_extra = [], []
        for i in sorted({max(M - 2, 0), M - 1}):
            r_extra.append(np.full(N, i, dtype=np.int64))
            c_extra.append(np.arange(N, dtype=np.int64))
        for j in sorted({max(N - 2, 0), N - 1}):
            r_extra.append(np.arange(M, dtype=np.int64))
            c_extra.append(np.full(M, j, dtype=np.int64))
        r_extra.append(np.array([0, 0, M - 1, M - 1], dtype=np.int64))
        c_extra.append(np.array([0, N - 1, 0, N - 1], dtype=np.int64))
        rows = np.concatenate([rows] + r_extra)
        cols = np.concatenate([cols] + c_extra)
    return rows, cols


def irregular_shapes(seed=20261202, count=16):
    """The seeded irregular bf16 sweep: M, N in [1000, 8192], K in [1000, 16384].

    Drawn with CPython's ``random.Random(seed)`` in the order M, N, K per
    shape; any value that is a multiple of 128 is redrawn.
    """
    rnd = random.Random(seed)

    def pick(lo, hi):
        while True:
            v = rnd.randint(lo, hi)
            if v % 128:
                return v

    shapes = []
    for _ in range(count):
        m = pick(1000, 8192)
        n = pick(1000, 8192)
        k = pick(1000, 16384)
        shapes.append((m, n, k))
    return shapes


# The five workloads: (name, M, N, K, dtype, distribution, scale, value seed).
def log_sampled_shapes(n, seed=20261203, lo=256, hi=8192, step=256):
    """n shapes (M, N, K), each dimension drawn log-uniformly in [lo, hi] and
    rounded to a multiple of step (seeded).  The Triton Stream-K issue's shape
    benchmark (its later revisions) takes the cube of a log-spaced grid of
    sizes over the same range, rounded to multiples of 256; this draws from
    the same distribution instead of walking the whole cube."""
    import math
    rnd = random.Random(seed)

    def one():
        v = math.exp(rnd.uniform(math.log(lo), math.log(hi)))
        return int(min(hi, max(lo, round(v / step) * step)))
    return [(one(), one(), one()) for _ in range(n)]


WORKLOADS = {
    "fp32_256": dict(M=256, N=256, K=256, dtype="f32", dist="uniform", scale=1.0, seed=101),
    "fp16_4096": dict(M=4096, N=4096, K=4096, dtype="f16", dist="normal", scale=1.0, seed=102),
    "fp16_1536x1536x8192": dict(M=1536, N=1536, K=8192, dtype="f16", dist="uniform", scale=1.0,
                                seed=103),
    "bf16_512x512x65536": dict(M=512, N=512, K=65536, dtype="bf16", dist="normal",
                               scale=1.0 / 256.0, seed=104),
    "bf16_8192x28672x8192": dict(M=8192, N=28672, K=8192, dtype="bf16", dist="normal", scale=1.0,
                                 seed=105),
}

# Beyond the workloads above: the int8 -> int32 path (the pages' kernel picks an
# int32 accumulator for int8), at the 4096^3 shape; integers uniform in [-128, 127].
EXTRA_WORKLOADS = {
    "i8_4096": dict(M=4096, N=4096, K=4096, dtype="i8", dist="int8", scale=1.0, seed=106),
}


def irregular_workloads():
    """The 16 irregular bf16 shapes as workload dicts (value seeds 1050 + j)."""
    return {f"bf16_irregular_{j:02d}_{m}x{n}x{k}": dict(M=m, N=n, K=k, dtype="bf16", dist="normal",
                                                         scale=1.0, seed=1050 + j)
            for j, (m, n, k) in enumerate(irregular_shapes())}
