"""Whole GEMM products for the full-size comparisons (test infrastructure only).

Only the tests, the smoke check and the benchmark may import this module; the
product path never does, and nothing here comes from the product path.

What it computes is the definition the triple loop in ``oracle_gemm.c``
writes out, C = A * B ("Hand-Written PTX Tensor-Core GEMM Kernels: A
Multi-Precision Study on NVIDIA L4": GEMM in FP16, INT8 and INT4, abstract
and Section I; D = AB + C with C = 0, Section II-A; INT32 results without
scaling, Section VI; operand roles of the .row.col MMA, Listing 2), with one
library step: the sum over k is a single fp64 matrix product (numpy).  That
makes a whole 8192^3 product take seconds rather than the triple loop's
minutes, so every element of a full-size output can be compared.

Why one fp64 matrix product is the definition here:
  * FP16: binary16 values convert to fp64 exactly, and a product of two of
    them (11 + 11 significant bits) is exact in fp64.  The matrix product sums
    the K exact products in some order; its error is below K * 2^-53 * S per
    element, with S = sum_k |a_ik b_kj| (the scale of the tolerance
    1e-3 * S), i.e. below 1e-12 * S for K <= 8192.  S is the same product of
    the absolute values.
  * INT8 / INT4: every product and every partial sum is an integer of
    magnitude at most K * 2^14 < 2^53 (the checked range), and such integers
    and their sums are exact in fp64 in any order, so the result is the exact
    integer sum.

Layouts (the library's operand contract):
    A   (M, lda)  row-major, the first K values of a row take part
    Bt  (N, ldb)  column-major B stored as its rows (rowb=False), or
    B   (K, ldb)  row-major B, the first N values of a row take part (rowb=True)
INT4 arrays hold bytes; element k of a row is byte k // 2, its low nibble for
even k and its high nibble for odd k, two's complement in [-8, 7] (rowb: the
same along N).
"""
from __future__ import annotations

import numpy as np

_EXACT_LIMIT = 2.0 ** 53


def s4_values(packed, count):
    """Signed 4-bit values of each row of a packed byte array, by the layout
    definition: element e of a row sits in byte e // 2, in the low nibble when
    e is even and in the high nibble when e is odd, as a two's complement
    4-bit value.  Returns int16 (rows, count)."""
    b = np.asarray(packed, dtype=np.uint8)
    nib = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int16)
    nib[:, 0::2] = b & 0x0F
    nib[:, 1::2] = b >> 4
    nib = np.where(nib < 8, nib, nib - 16)
    if count > nib.shape[1]:
        raise ValueError("fewer packed values than requested")
    return nib[:, :count]


def _operands_f64(A, B, K, N, rowb, decode):
    """(M, K) values of A and (K, N) values of B as fp64, cut to the extents."""
    a = decode(A, K)
    if rowb:
        b = decode(B, N)[:K]
        if b.shape[0] < K:
            raise ValueError("B holds fewer than K rows")
    else:
        b = decode(B, K)[:N].T
    return np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)


def _plain(width_of):
    def decode(x, count):
        x = np.asarray(x)
        if count > width_of(x):
            raise ValueError("fewer values per row than requested")
        return x[:, :count]
    return decode


def _dims(A, B, K, N, rowb, packed):
    width = lambda x: (2 * x.shape[1]) if packed else x.shape[1]
    K = width(np.asarray(A)) if K is None else K
    if N is None:
        N = width(np.asarray(B)) if rowb else np.asarray(B).shape[0]
    if K < 0 or N < 0:
        raise ValueError("negative extent")
    return K, N


def gemm_f16(A, B, K=None, N=None, rowb=False):
    """FP16 product in fp64: returns (R, S) with R = A * B and
    S = |A| * |B| (element-wise absolute values), each (M, N) float64."""
    K, N = _dims(A, B, K, N, rowb, False)
    a, b = _operands_f64(np.asarray(A, dtype=np.float16), np.asarray(B, dtype=np.float16),
                         K, N, rowb, _plain(lambda x: x.shape[1]))
    if K == 0:
        z = np.zeros((a.shape[0], N))
        return z, z.copy()
    if not (np.all(np.isfinite(a)) and np.all(np.isfinite(b))):
        raise ValueError("non-finite FP16 input")
    return a @ b, np.abs(a) @ np.abs(b)


def _integer(a, b, bound):
    if a.shape[1] * bound >= _EXACT_LIMIT:
        raise ValueError("sums could leave the range where fp64 is exact")
    if a.shape[1] == 0:
        return np.zeros((a.shape[0], b.shape[1]), np.int64)
    return np.rint(a @ b).astype(np.int64)


def gemm_i8(A, B, K=None, N=None, rowb=False):
    """INT8 product, exact, as int64 (M, N)."""
    K, N = _dims(A, B, K, N, rowb, False)
    a, b = _operands_f64(np.asarray(A, dtype=np.int8), np.asarray(B, dtype=np.int8),
                         K, N, rowb, _plain(lambda x: x.shape[1]))
    return _integer(a, b, 128.0 * 128.0)


def gemm_i4(A, B, K=None, N=None, rowb=False):
    """Packed INT4 product, exact, as int64 (M, N)."""
    K, N = _dims(A, B, K, N, rowb, True)
    a, b = _operands_f64(np.asarray(A, dtype=np.uint8), np.asarray(B, dtype=np.uint8),
                         K, N, rowb, s4_values)
    return _integer(a, b, 8.0 * 8.0)
