"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin_* function raises AssertionError when the oracle is wrong.  The
tests below run them against the committed oracle; test_oracle_mutants.py
runs them against deliberately broken copies of the oracle's C source to
show that every planted mistake is caught by at least one pin.

Sources of truth used here:
  * the worked 16x8x16 FP16 example printed in "PTX Programming from Your
    First Kernel to Tensor Cores", section "Multiply one tile with a full
    warp" (tests/golden/mma_lab_identity.json);
  * closed forms (all-ones, identities, the INT8 and INT4 extremes);
  * numpy's own binary16 decoder, on all 65536 bit patterns;
  * an independent pure-Python evaluator with exact integers and
    fractions.Fraction on every shape in {1..8}^3;
  * exhaustive product tables (every INT8 pair, every INT4 pair in both
    nibble positions) against numpy integer outer products;
  * algebraic invariants (transpose symmetry, linearity, thread-count
    independence, entry-wise vs full agreement).

The whole-product form in oracle/matmul.py (the same definition with the sum
over k done by one fp64 matrix product, used for full-size comparisons) is
pinned by the MATMUL_PINS: the worked example, closed forms, exact brute
force, product tables, and agreement with the pinned triple loop.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mma_lab_identity.json")


# --------------------------------------------------------------------------
# helpers that build operands by the layout definition (A row-major, B
# column-major stored as Bt rows, int4 low nibble = even k)

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _lab_operands(reverse_rows=False):
    g = _golden()
    M, N, K = g["M"], g["N"], g["K"]
    A = np.eye(M, K)
    if reverse_rows:
        A = A[::-1].copy()
    Bmat = np.array([[8 * r + c + 1 for c in range(N)] for r in range(K)], dtype=np.float64)
    return g, A, Bmat


# --------------------------------------------------------------------------
# pins

def pin_half_decoder():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the sign of zero matters for the S = 0 case
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def pin_mma_lab_f16():
    g, A, Bmat = _lab_operands()
    R, S = oracle.gemm_f16(A.astype(np.float16), Bmat.T.astype(np.float16))
    for r, c, v in g["printed_entries"]:
        assert R[r, c] == v, (r, c, R[r, c], v)
    assert np.array_equal(R, Bmat[: g["M"]])
    _, Ar, _ = _lab_operands(reverse_rows=True)
    R2, _ = oracle.gemm_f16(Ar.astype(np.float16), Bmat.T.astype(np.float16))
    assert list(R2[0]) == g["row_reversed_A_first_row"]


def pin_mma_lab_integer():
    # The same identity-reproduces-B construction with values that fit the
    # integer types (our adaptation of the printed FP16 example).
    g, A, _ = _lab_operands()
    M, N, K = g["M"], g["N"], g["K"]
    B8 = np.array([[8 * r + c - 64 for c in range(N)] for r in range(K)], dtype=np.int8)
    C = oracle.gemm_i8(A.astype(np.int8), np.ascontiguousarray(B8.T))
    assert np.array_equal(C, B8.astype(np.int64))
    B4 = np.array([[((8 * r + c) % 16) - 8 for c in range(N)] for r in range(K)], dtype=np.int8)
    C4 = oracle.gemm_i4(synth.pack_int4(A.astype(np.int8)), synth.pack_int4(np.ascontiguousarray(B4.T)))
    assert np.array_equal(C4, B4.astype(np.int64))
    _, Ar, _ = _lab_operands(reverse_rows=True)
    C4r = oracle.gemm_i4(synth.pack_int4(Ar.astype(np.int8)), synth.pack_int4(np.ascontiguousarray(B4.T)))
    assert np.array_equal(C4r, B4[::-1].astype(np.int64))


def pin_closed_forms():
    M, N, K = 5, 7, 34
    ones16 = np.ones((M, K), np.float16), np.ones((N, K), np.float16)
    R, S = oracle.gemm_f16(*ones16)
    assert np.all(R == K) and np.all(S == K)
    neg = np.full((M, K), -1.0, np.float16), np.ones((N, K), np.float16)
    R, S = oracle.gemm_f16(*neg)
    assert np.all(R == -K) and np.all(S == K)
    assert np.all(oracle.gemm_i8(np.ones((M, K), np.int8), np.ones((N, K), np.int8)) == K)
    assert np.all(oracle.gemm_i8(np.full((M, K), -128, np.int8), np.full((N, K), -128, np.int8)) == 16384 * K)
    assert np.all(oracle.gemm_i8(np.full((M, K), -128, np.int8), np.full((N, K), 127, np.int8)) == -16256 * K)
    p = synth.pack_int4
    assert np.all(oracle.gemm_i4(p(np.ones((M, K), np.int8)), p(np.ones((N, K), np.int8))) == K)
    assert np.all(oracle.gemm_i4(p(np.full((M, K), -8, np.int8)), p(np.full((N, K), -8, np.int8))) == 64 * K)
    assert np.all(oracle.gemm_i4(p(np.full((M, K), -8, np.int8)), p(np.full((N, K), 7, np.int8))) == -56 * K)
    # K = 0: the empty sum
    assert np.all(oracle.gemm_i8(np.ones((M, 16), np.int8), np.ones((N, 16), np.int8), K=0) == 0)
    R, S = oracle.gemm_f16(np.ones((M, 16), np.float16), np.ones((N, 16), np.float16), K=0)
    assert np.all(R == 0) and np.all(S == 0)


def pin_identities():
    rng = np.random.default_rng(7)
    M, K = 9, 12
    # B = I (K x K, column-major = its own transpose): C = A
    A8 = rng.integers(-128, 128, (M, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8(A8, np.eye(K, dtype=np.int8)), A8.astype(np.int64))
    A4 = rng.integers(-8, 8, (M, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i4(synth.pack_int4(A4), synth.pack_int4(np.eye(K, dtype=np.int8))),
                          A4.astype(np.int64))
    Ah = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    R, _ = oracle.gemm_f16(Ah, np.eye(K, dtype=np.float16))
    assert np.array_equal(R, Ah.astype(np.float64))
    # A = I: C = B, with a non-square B to fix which index is which
    N = 5
    Bt8 = rng.integers(-128, 128, (N, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8(np.eye(K, dtype=np.int8), Bt8), Bt8.T.astype(np.int64))


def _exact_eval(prec, A, Bt, K):
    """Independent evaluator: the definition with Python ints / Fractions."""
    M, N = A.shape[0], Bt.shape[0]
    if prec == "i4":
        Au = synth.unpack_int4(A).astype(int).tolist()
        Bu = synth.unpack_int4(Bt).astype(int).tolist()
    elif prec == "i8":
        Au, Bu = A.astype(int).tolist(), Bt.astype(int).tolist()
    else:
        Au = [[Fraction(float(v)) for v in row] for row in A]
        Bu = [[Fraction(float(v)) for v in row] for row in Bt]
    C = [[0] * N for _ in range(M)]
    S = [[0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = 0
            mag = 0
            for k in range(K):
                prod = Au[i][k] * Bu[j][k]
                acc += prod
                mag += abs(prod)
            C[i][j] = acc
            S[i][j] = mag
    return C, S


def _padded(x, ld, fill):
    return synth.with_leading_dim(x, ld, fill)


def pin_brute_force_tiny(shapes=None):
    rng = np.random.default_rng(11)
    if shapes is None:
        shapes = [(m, n, k) for m in range(1, 9) for n in range(1, 9) for k in range(1, 9)]
    for (m, n, k) in shapes:
        # leading dims larger than K, padded with values that would poison the sum
        a8 = rng.integers(-128, 128, (m, k), dtype=np.int8)
        b8 = rng.integers(-128, 128, (n, k), dtype=np.int8)
        C = oracle.gemm_i8(_padded(a8, k + 3, 127), _padded(b8, k + 5, -128), K=k)
        E, _ = _exact_eval("i8", a8, b8, k)
        assert C.tolist() == E, ("i8", m, n, k)

        k4 = 2 * k
        a4 = rng.integers(-8, 8, (m, k4), dtype=np.int8)
        b4 = rng.integers(-8, 8, (n, k4), dtype=np.int8)
        pa = _padded(synth.pack_int4(a4), k + 2, 0x77)
        pb = _padded(synth.pack_int4(b4), k + 1, 0x88)
        C4 = oracle.gemm_i4(pa, pb, K=k4)
        E4, _ = _exact_eval("i4", synth.pack_int4(a4), synth.pack_int4(b4), k4)
        assert C4.tolist() == E4, ("i4", m, n, k4)
        # odd K: the last byte's high nibble must be ignored
        if k4 > 2:
            C4o = oracle.gemm_i4(pa, pb, K=k4 - 1)
            E4o, _ = _exact_eval("i4", synth.pack_int4(a4), synth.pack_int4(b4), k4 - 1)
            assert C4o.tolist() == E4o, ("i4 odd", m, n, k4 - 1)

        ah = rng.uniform(-2, 2, (m, k)).astype(np.float16)
        bh = rng.uniform(-2, 2, (n, k)).astype(np.float16)
        R, S = oracle.gemm_f16(_padded(ah, k + 4, np.float16(np.nan)),
                               _padded(bh, k + 2, np.float16(np.inf)), K=k)
        Eh, Sh = _exact_eval("f16", ah, bh, k)
        for i in range(m):
            for j in range(n):
                assert np.isfinite(R[i, j]) and np.isfinite(S[i, j]), ("f16", m, n, k)
                # fp64 sequential summation error is below k * 2^-53 * S
                assert abs(Fraction(R[i, j]) - Eh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j], ("f16", m, n, k)
                assert abs(Fraction(S[i, j]) - Sh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j]


def pin_product_tables():
    # every INT8 pair: M = N = 256 rows/cols of one value each, K = 1
    v = np.arange(-128, 128, dtype=np.int8).reshape(256, 1)
    C = oracle.gemm_i8(v, v)
    assert np.array_equal(C, np.outer(v.astype(np.int64), v.astype(np.int64)))
    # every INT4 pair, in both nibble positions and crossed positions (K = 2)
    w = np.arange(-8, 8, dtype=np.int8)
    z = np.zeros(16, np.int8)
    even = synth.pack_int4(np.stack([w, z], axis=1))
    odd = synth.pack_int4(np.stack([z, w], axis=1))
    outer = np.outer(w.astype(np.int64), w.astype(np.int64))
    assert np.array_equal(oracle.gemm_i4(even, even), outer)
    assert np.array_equal(oracle.gemm_i4(odd, odd), outer)
    assert np.all(oracle.gemm_i4(even, odd) == 0)
    # a raw byte whose nibbles differ in sign: 0x8F = (k0 = -1, k1 = -8)
    a = np.array([[0x8F]], np.uint8)
    b = np.array([[0x12]], np.uint8)  # (k0 = 2, k1 = 1)
    assert oracle.gemm_i4(a, b)[0, 0] == (-1) * 2 + (-8) * 1


def pin_invariants():
    rng = np.random.default_rng(3)
    M, N, K = 13, 11, 37
    A = rng.integers(-128, 128, (M, K), dtype=np.int8)
    Bt = rng.integers(-128, 128, (N, K), dtype=np.int8)
    C = oracle.gemm_i8(A, Bt)
    # (A B)^T = B^T A^T: swapping the operand roles transposes the result
    assert np.array_equal(oracle.gemm_i8(Bt, A), C.T)
    # linearity in B
    B1 = rng.integers(-60, 60, (N, K), dtype=np.int8)
    B2 = rng.integers(-60, 60, (N, K), dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8(A, (B1 + B2).astype(np.int8)),
                          oracle.gemm_i8(A, B1) + oracle.gemm_i8(A, B2))
    # thread count does not change any bit, FP16 included
    Ah = rng.standard_normal((M, K)).astype(np.float16)
    Bh = rng.standard_normal((N, K)).astype(np.float16)
    R1, S1 = oracle.gemm_f16(Ah, Bh, threads=1)
    R7, S7 = oracle.gemm_f16(Ah, Bh, threads=7)
    assert np.array_equal(R1, R7) and np.array_equal(S1, S7)
    # entry-wise agrees with the full product
    rows = rng.integers(0, M, 20)
    cols = rng.integers(0, N, 20)
    assert np.array_equal(oracle.entries_i8(A, Bt, rows, cols), C[rows, cols])
    Re, Se = oracle.entries_f16(Ah, Bh, rows, cols)
    assert np.array_equal(Re, R1[rows, cols]) and np.array_equal(Se, S1[rows, cols])
    A4 = synth.pack_int4(rng.integers(-8, 8, (M, 2 * K), dtype=np.int8))
    B4 = synth.pack_int4(rng.integers(-8, 8, (N, 2 * K), dtype=np.int8))
    C4 = oracle.gemm_i4(A4, B4)
    assert np.array_equal(oracle.entries_i4(A4, B4, rows, cols), C4[rows, cols])
    assert np.array_equal(oracle.gemm_i4(B4, A4), C4.T)


def pin_half_rounding():
    """binary32 -> binary16 (round to nearest even) against numpy's IEEE conversion."""
    # every binary16 value converts to itself
    halves = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite = halves[np.isfinite(halves)]
    got = np.array([oracle.float_to_half(float(np.float32(h))) for h in finite], np.uint16)
    assert np.array_equal(got, finite.view(np.uint16))
    # every midpoint between consecutive positive binary16 values (exact in binary32): ties to even
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    for m in np.concatenate([mids, -mids]):
        assert oracle.float_to_half(float(m)) == np.float32(m).astype(np.float16).view(np.uint16), m
    # random binary32 values across the whole binary16 range, subnormals and overflow
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 17, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([65504, 65519.996, 65520, 65536, 1e30, -1e30, 2 ** -24, 2 ** -25,
                                       2 ** -26, 3 * 2 ** -26, 1e-30, 0.0, -0.0])])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, want)


def pin_dequant():
    """The dequantizing epilogue: ((float)S * scale_a[i]) * scale_b[j] in binary32."""
    rng = np.random.default_rng(9)
    M, N = 7, 5
    S = rng.integers(-2 ** 31, 2 ** 31, (M, N), dtype=np.int64)
    # unit scales give the sum rounded to binary32
    C = oracle.dequant(S, np.ones(M, np.float32), np.ones(N, np.float32))
    assert np.array_equal(C, S.astype(np.float32))
    # power-of-two scales are exact on sums below 2^24
    Ss = rng.integers(-2 ** 24, 2 ** 24, (M, N), dtype=np.int64)
    ea = rng.integers(-20, 20, M)
    eb = rng.integers(-20, 20, N)
    C = oracle.dequant(Ss, np.exp2(ea).astype(np.float32), np.exp2(eb).astype(np.float32))
    assert np.array_equal(C.astype(np.float64), Ss * np.exp2(ea)[:, None] * np.exp2(eb)[None, :])
    # arbitrary scales: the same three binary32 roundings, in the same order, done by numpy
    sa = rng.uniform(1e-3, 4, M).astype(np.float32)
    sb = rng.uniform(1e-3, 4, N).astype(np.float32)
    C = oracle.dequant(S, sa, sb)
    want = (S.astype(np.float32) * sa[:, None]) * sb[None, :]
    assert want.dtype == np.float32 and np.array_equal(C, want)
    # and within three roundings of the exact real product
    exact = S.astype(np.float64) * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :]
    assert np.all(np.abs(C - exact) <= 3 * 2.0 ** -24 * np.abs(exact))
    # binary16 output: the binary32 result rounded once more
    Sm = rng.integers(-2 ** 20, 2 ** 20, (M, N), dtype=np.int64)
    Ch = oracle.dequant(Sm, sa * 1e-3, sb, half_out=True)
    wanth = ((Sm.astype(np.float32) * (sa * np.float32(1e-3))[:, None]) * sb[None, :]).astype(np.float16)
    assert Ch.dtype == np.float16 and np.array_equal(Ch.view(np.uint16), wanth.view(np.uint16))
    # the elementwise form, with signed scales and zero sums (signed zeros are bit-exact)
    n = 4000
    Se = rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int64)
    Se[::7] = 0
    sae = (rng.uniform(-4, 4, n) * np.exp2(rng.integers(-30, 10, n))).astype(np.float32)
    sbe = (rng.uniform(-4, 4, n) * np.exp2(rng.integers(-30, 10, n))).astype(np.float32)
    want = (Se.astype(np.float32) * sae) * sbe
    got = oracle.dequant_entries(Se, sae, sbe)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    goth = oracle.dequant_entries(Se, sae, sbe, half_out=True)
    with np.errstate(over="ignore"):  # large products round to infinity, on both sides
        wanth = want.astype(np.float16)
    assert np.array_equal(goth.view(np.uint16), wanth.view(np.uint16))


def _exact_eval_rowb(prec, A, B, N, K):
    """Independent evaluator for B row-major: B[k][j], Python ints / Fractions."""
    M = A.shape[0]
    if prec == "i4":
        Au = synth.unpack_int4(A).astype(int).tolist()
        Bu = synth.unpack_int4(B).astype(int).tolist()
    elif prec == "i8":
        Au, Bu = A.astype(int).tolist(), B.astype(int).tolist()
    else:
        Au = [[Fraction(float(v)) for v in row] for row in A]
        Bu = [[Fraction(float(v)) for v in row] for row in B]
    C = [[sum((Au[i][k] * Bu[k][j] for k in range(K)), 0) for j in range(N)] for i in range(M)]
    S = [[sum((abs(Au[i][k] * Bu[k][j]) for k in range(K)), 0) for j in range(N)] for i in range(M)]
    return C, S


def pin_rowb():
    """B row-major (element (k, j) at B[k*ldb + j]; INT4 packed along N)."""
    # the PTX tutorial's worked example is stated with B as a K x N row-major matrix
    g, A, Bmat = _lab_operands()
    R, _ = oracle.gemm_f16_rowb(A.astype(np.float16), Bmat.astype(np.float16))
    for r, c, v in g["printed_entries"]:
        assert R[r, c] == v
    _, Ar, _ = _lab_operands(reverse_rows=True)
    R2, _ = oracle.gemm_f16_rowb(Ar.astype(np.float16), Bmat.astype(np.float16))
    assert list(R2[0]) == g["row_reversed_A_first_row"]
    M, N, K = g["M"], g["N"], g["K"]
    B8 = np.array([[8 * r + c - 64 for c in range(N)] for r in range(K)], dtype=np.int8)
    assert np.array_equal(oracle.gemm_i8_rowb(A.astype(np.int8), B8), B8.astype(np.int64))
    B4 = np.array([[((8 * r + c) % 16) - 8 for c in range(N)] for r in range(K)], dtype=np.int8)
    C4 = oracle.gemm_i4_rowb(synth.pack_int4(A.astype(np.int8)), synth.pack_int4(B4))
    assert np.array_equal(C4, B4.astype(np.int64))
    # INT4 nibble order along N: a one-hot A row picks one row of B, value by value
    w = np.arange(-8, 8, dtype=np.int8)
    Bw = synth.pack_int4(np.stack([w, np.zeros(16, np.int8), w[::-1]]))   # 3 rows x 16 columns
    for k, want in ((0, w), (1, np.zeros(16)), (2, w[::-1])):
        a = np.zeros((1, 4), np.int8)
        a[0, k] = 1
        assert np.array_equal(oracle.gemm_i4_rowb(synth.pack_int4(a), Bw, K=3)[0], want)
    a = synth.pack_int4(np.array([[0, 0, -3, 0]], np.int8))
    assert np.array_equal(oracle.gemm_i4_rowb(a, Bw, K=3)[0], -3 * w[::-1].astype(np.int64))
    # brute force on tiny shapes; columns past N and rows past K hold poison
    rng = np.random.default_rng(17)
    for m, n, k in [(m, n, k) for m in (1, 2, 5) for n in range(1, 7) for k in range(1, 7)]:
        b8 = rng.integers(-128, 128, (k, n), dtype=np.int8)
        a8 = rng.integers(-128, 128, (m, k), dtype=np.int8)
        b8p = np.vstack([_padded(b8, n + 3, 127), np.full((2, n + 3), -128, np.int8)])
        C = oracle.gemm_i8_rowb(_padded(a8, k + 1, 127), b8p, N=n, K=k)
        assert C.tolist() == _exact_eval_rowb("i8", a8, b8, n, k)[0], ("i8", m, n, k)
        n4 = 2 * n
        b4 = rng.integers(-8, 8, (k, n4), dtype=np.int8)
        a4 = rng.integers(-8, 8, (m, 2 * k), dtype=np.int8)
        b4p = np.vstack([_padded(synth.pack_int4(b4), n + 2, 0x77), np.full((2, n + 2), 0x88, np.uint8)])
        C4 = oracle.gemm_i4_rowb(_padded(synth.pack_int4(a4), k + 1, 0x77), b4p, N=n4, K=k)
        E4 = _exact_eval_rowb("i4", synth.pack_int4(a4), synth.pack_int4(b4), n4, k)[0]
        assert C4.tolist() == E4, ("i4", m, n4, k)
        if n4 > 1:   # odd N: the last byte's high nibble is outside
            C4o = oracle.gemm_i4_rowb(_padded(synth.pack_int4(a4), k + 1, 0x77), b4p, N=n4 - 1, K=k)
            assert C4o.tolist() == [row[:n4 - 1] for row in E4], ("i4 odd N", m, n4, k)
        bh = rng.uniform(-2, 2, (k, n)).astype(np.float16)
        ah = rng.uniform(-2, 2, (m, k)).astype(np.float16)
        bhp = np.vstack([_padded(bh, n + 2, np.float16(np.inf)),
                         np.full((1, n + 2), np.nan, np.float16)])
        R, S = oracle.gemm_f16_rowb(_padded(ah, k + 2, np.float16(np.nan)), bhp, N=n, K=k)
        Eh, Sh = _exact_eval_rowb("f16", ah, bh, n, k)
        for i in range(m):
            for j in range(n):
                assert abs(Fraction(R[i, j]) - Eh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j]
                assert abs(Fraction(S[i, j]) - Sh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j]
    # entry-wise forms agree with the full products
    A8, B8t = synth.operands("i8", 37, 45, 70, 3, 4)
    B8r = np.ascontiguousarray(B8t.T)
    full = oracle.gemm_i8_rowb(A8, B8r)
    rows, cols = rng.integers(0, 37, 50), rng.integers(0, 45, 50)
    assert np.array_equal(oracle.entries_i8_rowb(A8, B8r, rows, cols), full[rows, cols])
    A4, _ = synth.operands("i4", 37, 45, 70, 5, 6)
    B4r = synth.pack_int4(rng.integers(-8, 8, (70, 46), dtype=np.int8))
    full4 = oracle.gemm_i4_rowb(A4, B4r)
    assert np.array_equal(oracle.entries_i4_rowb(A4, B4r, rows, cols), full4[rows, cols])
    Ah, Bht = synth.operands("f16", 37, 45, 70, 7, 8)
    Bhr = np.ascontiguousarray(Bht.T)
    Rf, Sf = oracle.gemm_f16_rowb(Ah, Bhr)
    Re, Se = oracle.entries_f16_rowb(Ah, Bhr, rows, cols)
    assert np.array_equal(Re, Rf[rows, cols]) and np.array_equal(Se, Sf[rows, cols])



# --------------------------------------------------------------------------
# pins of the whole-product form (oracle/matmul.py: the same definition with
# the sum over k done by one fp64 matrix product), each taking that module so
# that planted mistakes in a copy of it can be run through them

def _lab_int_operands():
    g, A, _ = _lab_operands()
    M, N, K = g["M"], g["N"], g["K"]
    B8 = np.array([[8 * r + c - 64 for c in range(N)] for r in range(K)], dtype=np.int8)
    B4 = np.array([[((8 * r + c) % 16) - 8 for c in range(N)] for r in range(K)], dtype=np.int8)
    return g, A, B8, B4


def pin_matmul_lab(mm):
    """The PTX tutorial's printed example, with B in both layouts."""
    g, A, Bmat = _lab_operands()
    for R, _ in (mm.gemm_f16(A.astype(np.float16), Bmat.T.astype(np.float16)),
                 mm.gemm_f16(A.astype(np.float16), Bmat.astype(np.float16), rowb=True)):
        for r, c, v in g["printed_entries"]:
            assert R[r, c] == v, (r, c, R[r, c], v)
        assert np.array_equal(R, Bmat[: g["M"]])
    _, Ar, _ = _lab_operands(reverse_rows=True)
    R2, _ = mm.gemm_f16(Ar.astype(np.float16), Bmat.T.astype(np.float16))
    assert list(R2[0]) == g["row_reversed_A_first_row"]
    R3, _ = mm.gemm_f16(Ar.astype(np.float16), Bmat.astype(np.float16), rowb=True)
    assert list(R3[0]) == g["row_reversed_A_first_row"]
    g, A, B8, B4 = _lab_int_operands()
    assert np.array_equal(mm.gemm_i8(A.astype(np.int8), np.ascontiguousarray(B8.T)), B8.astype(np.int64))
    assert np.array_equal(mm.gemm_i8(A.astype(np.int8), B8, rowb=True), B8.astype(np.int64))
    pa = synth.pack_int4(A.astype(np.int8))
    assert np.array_equal(mm.gemm_i4(pa, synth.pack_int4(np.ascontiguousarray(B4.T))), B4.astype(np.int64))
    assert np.array_equal(mm.gemm_i4(pa, synth.pack_int4(B4), rowb=True), B4.astype(np.int64))
    _, Ar, _ = _lab_operands(reverse_rows=True)
    C4r = mm.gemm_i4(synth.pack_int4(Ar.astype(np.int8)), synth.pack_int4(np.ascontiguousarray(B4.T)))
    assert np.array_equal(C4r, B4[::-1].astype(np.int64))


def pin_matmul_closed_forms(mm):
    M, N, K = 5, 7, 34
    R, S = mm.gemm_f16(np.ones((M, K), np.float16), np.ones((N, K), np.float16))
    assert np.all(R == K) and np.all(S == K)
    R, S = mm.gemm_f16(np.full((M, K), -1.0, np.float16), np.ones((N, K), np.float16))
    assert np.all(R == -K) and np.all(S == K)
    R, S = mm.gemm_f16(np.full((M, K), -0.5, np.float16), np.full((K, N), 2.0, np.float16), rowb=True)
    assert np.all(R == -K) and np.all(S == K)
    assert np.all(mm.gemm_i8(np.full((M, K), -128, np.int8), np.full((N, K), -128, np.int8)) == 16384 * K)
    assert np.all(mm.gemm_i8(np.full((M, K), -128, np.int8), np.full((N, K), 127, np.int8)) == -16256 * K)
    p = synth.pack_int4
    assert np.all(mm.gemm_i4(p(np.full((M, K), -8, np.int8)), p(np.full((N, K), -8, np.int8))) == 64 * K)
    assert np.all(mm.gemm_i4(p(np.full((M, K), -8, np.int8)), p(np.full((N, K), 7, np.int8))) == -56 * K)
    assert np.all(mm.gemm_i4(p(np.full((M, K), 7, np.int8)), p(np.full((K, 2 * N), -8, np.int8)),
                             N=2 * N, rowb=True) == -56 * K)
    # K = 0: the empty sum
    assert np.all(mm.gemm_i8(np.ones((M, 16), np.int8), np.ones((N, 16), np.int8), K=0) == 0)
    R, S = mm.gemm_f16(np.ones((M, 16), np.float16), np.ones((N, 16), np.float16), K=0)
    assert R.shape == (M, N) and np.all(R == 0) and np.all(S == 0)


def pin_matmul_brute_force(mm):
    """Exact Python evaluation on tiny shapes, padding filled with poison, both B layouts."""
    rng = np.random.default_rng(23)
    for (m, n, k) in [(m, n, k) for m in (1, 2, 5, 8) for n in (1, 3, 7) for k in (1, 2, 5, 8)]:
        a8 = rng.integers(-128, 128, (m, k), dtype=np.int8)
        b8 = rng.integers(-128, 128, (n, k), dtype=np.int8)
        E, _ = _exact_eval("i8", a8, b8, k)
        assert mm.gemm_i8(_padded(a8, k + 3, 127), _padded(b8, k + 5, -128), K=k).tolist() == E
        b8r = np.vstack([_padded(np.ascontiguousarray(b8.T), n + 2, 127), np.full((2, n + 2), -128, np.int8)])
        assert mm.gemm_i8(_padded(a8, k + 1, 127), b8r, K=k, N=n, rowb=True).tolist() == E
        k4 = 2 * k
        a4 = rng.integers(-8, 8, (m, k4), dtype=np.int8)
        b4 = rng.integers(-8, 8, (n, k4), dtype=np.int8)
        pa = _padded(synth.pack_int4(a4), k + 2, 0x77)
        pb = _padded(synth.pack_int4(b4), k + 1, 0x88)
        E4, _ = _exact_eval("i4", synth.pack_int4(a4), synth.pack_int4(b4), k4)
        assert mm.gemm_i4(pa, pb, K=k4).tolist() == E4
        if k4 > 2:   # odd K: the last byte's high nibble stays out
            E4o, _ = _exact_eval("i4", synth.pack_int4(a4), synth.pack_int4(b4), k4 - 1)
            assert mm.gemm_i4(pa, pb, K=k4 - 1).tolist() == E4o
        n4 = 2 * n
        b4r = rng.integers(-8, 8, (k, n4), dtype=np.int8)
        a4k = rng.integers(-8, 8, (m, 2 * k), dtype=np.int8)
        b4rp = np.vstack([_padded(synth.pack_int4(b4r), n + 2, 0x77), np.full((2, n + 2), 0x88, np.uint8)])
        E4r = _exact_eval_rowb("i4", synth.pack_int4(a4k), synth.pack_int4(b4r), n4, k)[0]
        got = mm.gemm_i4(_padded(synth.pack_int4(a4k), k + 1, 0x77), b4rp, K=k, N=n4, rowb=True)
        assert got.tolist() == E4r
        if n4 > 1:   # odd N: the last byte's high nibble stays out
            got = mm.gemm_i4(_padded(synth.pack_int4(a4k), k + 1, 0x77), b4rp, K=k, N=n4 - 1, rowb=True)
            assert got.tolist() == [row[:n4 - 1] for row in E4r]
        ah = rng.uniform(-2, 2, (m, k)).astype(np.float16)
        bh = rng.uniform(-2, 2, (n, k)).astype(np.float16)
        Eh, Sh = _exact_eval("f16", ah, bh, k)
        R, S = mm.gemm_f16(_padded(ah, k + 4, np.float16(np.nan)), _padded(bh, k + 2, np.float16(np.inf)), K=k)
        bhr = np.vstack([_padded(np.ascontiguousarray(bh.T), n + 2, np.float16(np.inf)),
                         np.full((1, n + 2), np.nan, np.float16)])
        Rr, Sr = mm.gemm_f16(_padded(ah, k + 2, np.float16(np.nan)), bhr, K=k, N=n, rowb=True)
        for i in range(m):
            for j in range(n):
                for RR, SS in ((R, S), (Rr, Sr)):
                    assert abs(Fraction(RR[i, j]) - Eh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j], ("f16", m, n, k)
                    assert abs(Fraction(SS[i, j]) - Sh[i][j]) <= Fraction(k, 2 ** 52) * Sh[i][j]


def pin_matmul_product_tables(mm):
    v = np.arange(-128, 128, dtype=np.int8).reshape(256, 1)
    assert np.array_equal(mm.gemm_i8(v, v), np.outer(v.astype(np.int64), v.astype(np.int64)))
    w = np.arange(-8, 8, dtype=np.int8)
    z = np.zeros(16, np.int8)
    even = synth.pack_int4(np.stack([w, z], axis=1))
    odd = synth.pack_int4(np.stack([z, w], axis=1))
    outer = np.outer(w.astype(np.int64), w.astype(np.int64))
    assert np.array_equal(mm.gemm_i4(even, even), outer)
    assert np.array_equal(mm.gemm_i4(odd, odd), outer)
    assert np.all(mm.gemm_i4(even, odd) == 0)
    a = np.array([[0x8F]], np.uint8)   # (k0 = -1, k1 = -8)
    b = np.array([[0x12]], np.uint8)   # (k0 = 2, k1 = 1)
    assert mm.gemm_i4(a, b)[0, 0] == (-1) * 2 + (-8) * 1


def pin_matmul_matches_triple_loop(mm):
    """Against the pinned triple loop of oracle_gemm.c on multi-row random shapes."""
    for prec, (M, N, K) in (("f16", (37, 45, 300)), ("i8", (40, 33, 517)), ("i4", (29, 50, 402))):
        A, Bt = synth.operands(prec, M, N, K, 101, 102)
        if prec == "f16":
            R, S = oracle.gemm_f16(A, Bt, K=K)
            for B, rowb in ((Bt, False), (np.ascontiguousarray(Bt.T), True)):
                Rm, Sm = mm.gemm_f16(A, B, K=K, N=N, rowb=rowb)
                assert np.all(np.abs(Rm - R) <= 2 * K * 2.0 ** -53 * S)
                assert np.all(np.abs(Sm - S) <= 2 * K * 2.0 ** -53 * S)
        elif prec == "i8":
            C = oracle.gemm_i8(A, Bt, K=K)
            assert np.array_equal(mm.gemm_i8(A, Bt, K=K), C)
            assert np.array_equal(mm.gemm_i8(A, np.ascontiguousarray(Bt.T), K=K, N=N, rowb=True), C)
        else:
            C = oracle.gemm_i4(A, Bt, K=K)
            assert np.array_equal(mm.gemm_i4(A, Bt, K=K), C)
            Br = synth.pack_int4(np.ascontiguousarray(synth.unpack_int4(Bt)[:, :K].T))
            assert np.array_equal(mm.gemm_i4(A, Br, K=K, N=N, rowb=True), C)


MATMUL_PINS = [pin_matmul_lab, pin_matmul_closed_forms, pin_matmul_brute_force,
               pin_matmul_product_tables, pin_matmul_matches_triple_loop]


PINS = [pin_half_decoder, pin_mma_lab_f16, pin_mma_lab_integer, pin_closed_forms,
        pin_identities, pin_brute_force_tiny, pin_product_tables, pin_invariants,
        pin_half_rounding, pin_dequant, pin_rowb]


# --------------------------------------------------------------------------
# tests

@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(oracle_lib, pin):
    pin()


@pytest.mark.parametrize("pin", MATMUL_PINS, ids=[p.__name__ for p in MATMUL_PINS])
def test_matmul_pin(oracle_lib, pin):
    import oracle.matmul
    pin(oracle.matmul)


def test_rejects_bad_arguments(oracle_lib):
    with pytest.raises(ValueError):
        oracle.gemm_i8(np.ones((2, 4), np.int8), np.ones((2, 4), np.int8), K=-1)


def test_synth_stream_matches_scalar_definition():
    # vectorised SplitMix64 against the plain big-int definition
    for seed in (0, 1, 1234567, (3 << 32) ^ (8192 << 8) ^ 2):
        assert synth.splitmix64(seed, 64).tolist() == synth.splitmix64_scalar(seed, 64)
    # offset streams are slices of the same stream
    full = synth.splitmix64(99, 100)
    assert np.array_equal(synth.splitmix64(99, 40, start=60), full[60:])
    # commonly published first outputs of SplitMix64 for seed 1234567
    assert synth.splitmix64_scalar(1234567, 5) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_synth_distributions():
    a = synth.int8_matrix(256, 256, 5)
    assert a.min() == -128 and a.max() == 127 and abs(float(a.mean())) < 1.0
    v = synth.int4_values(128, 128, 6)
    assert v.min() == -8 and v.max() == 7
    assert np.array_equal(synth.unpack_int4(synth.pack_int4(v)), v)
    u = synth.f16_uniform(256, 256, 7).astype(np.float64)
    assert u.min() >= -1.0 and u.max() <= 1.0 and abs(u.mean()) < 0.01
    n = synth.f16_normal(256, 256, 8, 1.0).astype(np.float64)
    assert abs(n.mean()) < 0.02 and abs(n.std() - 1.0) < 0.02
    # pack order: low nibble holds the even k
    assert synth.pack_int4(np.array([[1, -1]], np.int8))[0, 0] == 0xF1


def test_synth_scales():
    s = synth.f32_scales(200000, 11, lo=-12, hi=-2)
    assert s.dtype == np.float32 and np.all(s >= 2.0 ** -12) and np.all(s < 2.0 ** -2)
    e = np.floor(np.log2(s.astype(np.float64))).astype(int)
    counts = np.bincount(e + 12, minlength=10)
    assert counts.size == 10 and np.all(np.abs(counts / s.size - 0.1) < 0.01)  # log-uniform
    assert np.array_equal(s, synth.f32_scales(200000, 11, lo=-12, hi=-2))
    assert not np.array_equal(s[:100], synth.f32_scales(100, 12))
    with pytest.raises(ValueError):
        synth.f32_scales(4, 0, lo=-130, hi=0)
