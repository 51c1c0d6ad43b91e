"""CPU reference oracle for C = A.B -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never imports, links or runs it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, ascending-k sums); this
module only compiles it with gcc and marshals numpy arrays through ctypes.
Inputs are raw bit patterns: ``uint32``/``float32`` for fp32, ``uint16`` for
fp16 and bf16, ``int8`` for int8, exactly as the GPU reads them.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}

_lib = None


def build(out=LIB, src=SRC, extra_flags=()):
    """Compile the oracle with gcc (no -ffast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           *extra_flags, src, "-o", out + ".tmp", "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path=LIB):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
    lib.oracle_gemm_full.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, dp, dp, ctypes.c_int]
    lib.oracle_gemm_full.restype = ctypes.c_int
    lib.oracle_gemm_sampled.argtypes = [ctypes.c_int, i64, i64, i64, vp, vp, i64,
                                        ctypes.POINTER(i64), ctypes.POINTER(i64), dp, dp,
                                        ctypes.c_int]
    lib.oracle_gemm_sampled.restype = ctypes.c_int
    lib.oracle_decode_array.argtypes = [ctypes.c_int, vp, i64, dp]
    lib.oracle_decode_array.restype = ctypes.c_int
    if path == LIB:
        _lib = lib
    return lib


def _bits(x, dtype):
    want = {"f32": np.uint32, "i8": np.int8}.get(dtype, np.uint16)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint8 and dtype == "i8":
        x = x.view(np.int8)
    if x.dtype == np.float32 and dtype == "f32":
        x = x.view(np.uint32)
    if x.dtype == np.float16 and dtype == "f16":
        x = x.view(np.uint16)
    if x.dtype != want:
        raise TypeError(f"{dtype} operand must hold {want.__name__} bit patterns, got {x.dtype}")
    return x


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def decode(x, dtype, lib=None):
    """Decode raw bit patterns to float64 with the oracle's own decoder."""
    lib = lib or load()
    x = _bits(x, dtype)
    out = np.empty(x.size, dtype=np.float64)
    rc = lib.oracle_decode_array(DTYPES[dtype], x.ctypes.data, x.size, _dptr(out))
    if rc:
        raise RuntimeError(f"oracle_decode_array failed ({rc})")
    return out.reshape(x.shape)


def gemm(a, b, dtype, nthreads=None, want_s=True, lib=None):
    """Full oracle: returns (C, S) as float64 M x N arrays (S None if not wanted)."""
    lib = lib or load()
    a, b = _bits(a, dtype), _bits(b, dtype)
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    # NaN-filled so an element the oracle failed to write cannot pass a check
    C = np.full((M, N), np.nan, dtype=np.float64)
    S = np.full((M, N), np.nan, dtype=np.float64) if want_s else None
    rc = lib.oracle_gemm_full(DTYPES[dtype], M, N, K, a.ctypes.data, b.ctypes.data,
                              _dptr(C), _dptr(S), nthreads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_gemm_full failed ({rc})")
    return C, S


def gemm_sampled(a, b, dtype, rows, cols, nthreads=None, lib=None):
    """Sampled oracle: (C[s], S[s]) for output elements (rows[s], cols[s])."""
    lib = lib or load()
    a, b = _bits(a, dtype), _bits(b, dtype)
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    n = rows.size
    C = np.full(n, np.nan, dtype=np.float64)
    S = np.full(n, np.nan, dtype=np.float64)
    p64 = ctypes.POINTER(ctypes.c_int64)
    rc = lib.oracle_gemm_sampled(DTYPES[dtype], M, N, K, a.ctypes.data, b.ctypes.data, n,
                                 rows.ctypes.data_as(p64), cols.ctypes.data_as(p64),
                                 _dptr(C), _dptr(S), nthreads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_gemm_sampled failed ({rc})")
    return C, S
