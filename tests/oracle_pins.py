"""Pins that tie the CPU oracle to facts other than itself.

Each function takes a loaded oracle library (``oracle.load(path)``) and raises
AssertionError when the oracle disagrees with:

* a library decoder (numpy's IEEE half, float32 reinterpretation),
* exact rational arithmetic on tiny shapes (Python ``fractions``),
* a product worked by hand (tests/golden/hand_product_2x3x2.json),
* identity / permutation matrices, small-integer inputs (int64 matmul),
* closed forms (all-ones, rank one, the i+k / k-j polynomial),
* algebraic invariants (transposition, power-of-two scaling),
* numpy's float64 matmul within the summation bound,
* itself across modes only where the definition says the bits must agree
  (sampled vs full, thread count, S against |A|.|B|).

tests/test_oracle_mutants.py plants plausible mistakes in a copy of oracle.c
and checks that every one of them trips at least one pin.
"""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
from persistent_stream_tiling_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U53 = 2.0 ** -53


def np_decode(bits, dtype):
    """Independent decoder: numpy's IEEE half and float32 reinterpretation."""
    bits = np.asarray(bits)
    with np.errstate(invalid="ignore"):
        return _np_decode(bits, dtype)


def _np_decode(bits, dtype):
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def exact_bits(values, dtype):
    """Bits of values that are exactly representable in ``dtype`` (checked)."""
    v32 = np.asarray(values, dtype=np.float32)
    bits = inputs.to_bits(v32, dtype)
    back = np_decode(bits, dtype)
    assert np.array_equal(back, np.asarray(values, dtype=np.float64)), "value not exact in dtype"
    return bits


def same_bits(x, y):
    return np.array_equal(np.asarray(x).view(np.uint64), np.asarray(y).view(np.uint64))


def pin_decode_f16_all(lib):
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(pats, "f16", lib=lib)
    ref = np_decode(pats, "f16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert same_bits(got[~nan], ref[~nan])


def pin_decode_bf16_all(lib):
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(pats, "bf16", lib=lib)
    ref = np_decode(pats, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert same_bits(got[~nan], ref[~nan])


def pin_decode_f32_sample(lib):
    rng = np.random.Generator(np.random.PCG64(7))
    pats = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 1, 0x7FFFFF, 0x800000, 0x3F800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000,
                        0x7FC00000, 0x80000001, 0x80000000], dtype=np.uint32)
    pats = np.concatenate([pats, special])
    got = oracle.decode(pats, "f32", lib=lib)
    ref = np_decode(pats, "f32")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert same_bits(got[~nan], ref[~nan])


def pin_hand_worked(lib):
    g = json.load(open(os.path.join(GOLDEN, "hand_product_2x3x2.json")))
    for dtype in ("f32", "f16", "bf16"):
        for a_key, c_key, s_key in (("A", "C", "S"), ("A_neg", "C_neg", "S_neg")):
            a = exact_bits(np.array(g[a_key], dtype=np.float64), dtype)
            b = exact_bits(np.array(g["B"], dtype=np.float64), dtype)
            C, S = oracle.gemm(a, b, dtype, lib=lib)
            assert np.array_equal(C, np.array(g[c_key], dtype=np.float64)), (dtype, a_key, C)
            assert np.array_equal(S, np.array(g[s_key], dtype=np.float64)), (dtype, a_key, S)


def pin_rational_tiny(lib):
    rng = np.random.Generator(np.random.PCG64(11))
    for dtype in ("f32", "f16", "bf16"):
        for case in range(40):
            M, N, K = (int(v) for v in rng.integers(1, 9, size=3))
            scale = 2.0 ** float(rng.integers(-6, 7))
            a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32) * scale, dtype)
            b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), dtype)
            av, bv = np_decode(a, dtype), np_decode(b, dtype)
            C, S = oracle.gemm(a, b, dtype, lib=lib)
            for i in range(M):
                for j in range(N):
                    ex = sum((Fraction(float(av[i, k])) * Fraction(float(bv[k, j]))
                              for k in range(K)), Fraction(0))
                    ex_s = sum((abs(Fraction(float(av[i, k]))) * abs(Fraction(float(bv[k, j])))
                                for k in range(K)), Fraction(0))
                    bound = Fraction(K) * Fraction(U53) * ex_s
                    assert abs(Fraction(float(C[i, j])) - ex) <= bound, (dtype, case, i, j)
                    assert abs(Fraction(float(S[i, j])) - ex_s) <= bound, (dtype, case, i, j)


def pin_identity_permutation(lib):
    rng = np.random.Generator(np.random.PCG64(13))
    for dtype in ("f32", "f16", "bf16"):
        M, K, N = 23, 17, 19
        a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32), dtype)
        b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), dtype)
        eye_k = exact_bits(np.eye(K), dtype)
        eye_m = exact_bits(np.eye(M), dtype)
        C, _ = oracle.gemm(a, eye_k, dtype, lib=lib)
        assert same_bits(C, np_decode(a, dtype))
        C, _ = oracle.gemm(eye_k, b, dtype, lib=lib)
        assert same_bits(C, np_decode(b, dtype))
        perm = rng.permutation(M)
        P = np.zeros((M, M))
        P[np.arange(M), perm] = 1.0
        am = inputs.to_bits(rng.standard_normal((M, N)).astype(np.float32), dtype)
        C, _ = oracle.gemm(exact_bits(P, dtype), am, dtype, lib=lib)
        assert same_bits(C, np_decode(am, dtype)[perm])
        C, _ = oracle.gemm(eye_m, am, dtype, lib=lib)
        assert same_bits(C, np_decode(am, dtype))


def pin_small_integers(lib):
    rng = np.random.Generator(np.random.PCG64(17))
    for dtype in ("f32", "f16", "bf16"):
        M, N, K = 37, 29, 513
        ai = rng.integers(-4, 5, size=(M, K))
        bi = rng.integers(-4, 5, size=(K, N))
        C, S = oracle.gemm(exact_bits(ai, dtype), exact_bits(bi, dtype), dtype, lib=lib)
        assert np.array_equal(C, (ai @ bi).astype(np.float64))
        assert np.array_equal(S, (np.abs(ai) @ np.abs(bi)).astype(np.float64))
    # long K through the sampled path: every partial sum stays an exact integer
    M, N, K = 5, 7, 65536
    ai = rng.integers(-4, 5, size=(M, K))
    bi = rng.integers(-4, 5, size=(K, N))
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    C, S = oracle.gemm_sampled(exact_bits(ai, "bf16"), exact_bits(bi, "bf16"), "bf16",
                               rows.ravel(), cols.ravel(), lib=lib)
    assert np.array_equal(C, (ai @ bi).astype(np.float64).ravel())
    assert np.array_equal(S, (np.abs(ai) @ np.abs(bi)).astype(np.float64).ravel())


def pin_closed_forms(lib):
    for dtype in ("f32", "f16", "bf16"):
        M, N, K = 9, 11, 300
        C, S = oracle.gemm(exact_bits(np.ones((M, K)), dtype), exact_bits(np.ones((K, N)), dtype),
                           dtype, lib=lib)
        assert np.all(C == K) and np.all(S == K)
        # rank one: a[i][k] = u_i, b[k][j] = v_j  ->  C = K u_i v_j (dyadic, exact)
        u = np.array([0.5, -1.5, 2.0, 0.25, -3.0, 1.0, 0.75, -0.125, 4.0])
        v = np.array([1.0, -2.0, 0.5, 3.0, -0.25, 1.5, -1.0, 2.5, 0.375, -4.0, 0.0625])
        C, _ = oracle.gemm(exact_bits(np.repeat(u[:, None], K, 1), dtype),
                           exact_bits(np.repeat(v[None, :], K, 0), dtype), dtype, lib=lib)
        assert np.array_equal(C, K * np.outer(u, v))
    # a[i][k] = i + k, b[k][j] = k - j:
    # C_ij = sum_k (i+k)(k-j) = -K i j + (i - j) K(K-1)/2 + (K-1)K(2K-1)/6
    for dtype, K in (("f32", 200), ("f16", 120), ("bf16", 100)):
        M, N = 13, 10
        i = np.arange(M)[:, None]
        j = np.arange(N)[None, :]
        a = exact_bits(np.arange(M)[:, None] + np.arange(K)[None, :], dtype)
        b = exact_bits(np.arange(K)[:, None] - np.arange(N)[None, :], dtype)
        C, _ = oracle.gemm(a, b, dtype, lib=lib)
        ref = -K * i * j + (i - j) * (K * (K - 1) // 2) + (K - 1) * K * (2 * K - 1) // 6
        assert np.array_equal(C, ref.astype(np.float64)), dtype


def pin_invariants(lib):
    rng = np.random.Generator(np.random.PCG64(19))
    M, N, K = 21, 14, 33
    a32 = rng.standard_normal((M, K)).astype(np.float32)
    b32 = rng.standard_normal((K, N)).astype(np.float32)
    a, b = inputs.to_bits(a32, "f32"), inputs.to_bits(b32, "f32")
    C, S = oracle.gemm(a, b, "f32", lib=lib)
    # transposition: (A.B)^T = B^T.A^T, same k order, so bitwise
    Ct, St = oracle.gemm(np.ascontiguousarray(b.T), np.ascontiguousarray(a.T), "f32", lib=lib)
    assert same_bits(Ct, np.ascontiguousarray(C.T)) and same_bits(St, np.ascontiguousarray(S.T))
    # power-of-two scaling is exact
    C2, _ = oracle.gemm(inputs.to_bits(a32 * np.float32(2.0), "f32"), b, "f32", lib=lib)
    assert same_bits(C2, 2.0 * C)
    # S is the product of the absolute values
    Cabs, _ = oracle.gemm(inputs.to_bits(np.abs(a32), "f32"), inputs.to_bits(np.abs(b32), "f32"),
                          "f32", lib=lib)
    assert same_bits(Cabs, S)
    # negating B negates C exactly
    Cn, _ = oracle.gemm(a, inputs.to_bits(-b32, "f32"), "f32", lib=lib)
    assert same_bits(Cn, -C)


def pin_numpy_crosscheck(lib):
    rng = np.random.Generator(np.random.PCG64(23))
    for dtype in ("f32", "f16", "bf16"):
        M, N, K = 31, 45, 1000
        a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32), dtype)
        b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), dtype)
        C, S = oracle.gemm(a, b, dtype, lib=lib)
        ref = np_decode(a, dtype) @ np_decode(b, dtype)
        assert np.all(np.abs(C - ref) <= 2 * K * U53 * S), dtype


def pin_sampled_matches_full(lib):
    rng = np.random.Generator(np.random.PCG64(29))
    for dtype in ("f32", "f16", "bf16"):
        M, N, K = 40, 24, 77
        a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32), dtype)
        b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), dtype)
        C, S = oracle.gemm(a, b, dtype, lib=lib)
        rows, cols = inputs.sample_positions(M, N, 200, seed=3, tails=True)
        Cs, Ss = oracle.gemm_sampled(a, b, dtype, rows, cols, lib=lib)
        assert same_bits(Cs, C[rows, cols]) and same_bits(Ss, S[rows, cols])


def pin_thread_invariance(lib):
    rng = np.random.Generator(np.random.PCG64(31))
    M, N, K = 29, 18, 150
    a = inputs.to_bits(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    b = inputs.to_bits(rng.standard_normal((K, N)).astype(np.float32), "bf16")
    C1, S1 = oracle.gemm(a, b, "bf16", nthreads=1, lib=lib)
    C7, S7 = oracle.gemm(a, b, "bf16", nthreads=7, lib=lib)
    assert same_bits(C1, C7) and same_bits(S1, S7)
    assert not np.isnan(C1).any()


def pin_int8(lib):
    # int8 (the final revision's int32-accumulator branch): every value and
    # every sum is an exact integer, so C must equal plain Python integer sums
    every = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(oracle.decode(every, "i8", lib=lib), every.astype(np.float64))
    rng = np.random.Generator(np.random.PCG64(37))
    for (M, N, K) in ((1, 1, 1), (3, 4, 5), (7, 2, 9), (5, 6, 33)):
        a = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        b = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
        C, S = oracle.gemm(a, b, "i8", lib=lib)
        for i in range(M):
            for j in range(N):
                assert C[i, j] == sum(int(a[i, k]) * int(b[k, j]) for k in range(K))
                assert S[i, j] == sum(abs(int(a[i, k])) * abs(int(b[k, j])) for k in range(K))
    # extremes: (-128)(-128) summed K times, and 127 * -128
    K = 4097
    C, _ = oracle.gemm(np.full((2, K), -128, np.int8), np.full((K, 3), -128, np.int8), "i8",
                       lib=lib)
    assert np.all(C == 16384 * K)
    C, _ = oracle.gemm(np.full((2, K), 127, np.int8), np.full((K, 3), -128, np.int8), "i8",
                       lib=lib)
    assert np.all(C == -16256 * K)
    # the sampled path on a long K: exact int64 sums
    M, N, K = 4, 5, 70000
    a = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-128, 128, size=(K, N)).astype(np.int8)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Cs, _ = oracle.gemm_sampled(a, b, "i8", rows.ravel(), cols.ravel(), lib=lib)
    assert np.array_equal(Cs, (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64).ravel())


ALL_PINS = [
    pin_decode_f16_all, pin_decode_bf16_all, pin_decode_f32_sample, pin_hand_worked,
    pin_rational_tiny, pin_identity_permutation, pin_small_integers, pin_closed_forms,
    pin_invariants, pin_numpy_crosscheck, pin_sampled_matches_full, pin_thread_invariance,
    pin_int8,
]
