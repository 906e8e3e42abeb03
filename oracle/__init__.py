"""CPU oracle for the multi-precision square GEMM (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never does, and the oracle never imports the product path: the two share
nothing but the seeded inputs from ``synth``.

The arithmetic lives in ``oracle_gemm.c`` (a plain triple loop, int64
accumulation for integers, fp64 for FP16); this module only marshals numpy
arrays into it.  Arrays follow the library's operand contract:

    A   (M, lda)   row-major, K contiguous            (int4: (M, lda/2) uint8)
    Bt  (N, ldb)   column-major B stored as its rows  (int4: (N, ldb/2) uint8)

and the first K elements of each row take part in the product.  The *_rowb
functions take B row-major instead, as a (K, ldb) array (int4: (K, ldb/2)
bytes packed along N), of which the first N columns take part.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle_gemm.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c into liboracle.so with the host C compiler."""
    if force or not os.path.exists(LIBRARY):
        tmp = LIBRARY + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", SOURCE, "-lm", "-o", tmp])
        os.replace(tmp, LIBRARY)
    return LIBRARY


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        lib = ctypes.CDLL(LIBRARY)
        i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_gemm_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, i32]
        lib.oracle_gemm_i8.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32]
        lib.oracle_gemm_i4.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32]
        lib.oracle_entries_f16.argtypes = [i64, p, i64, p, i64, i64, p, p, p, p]
        lib.oracle_entries_i8.argtypes = [i64, p, i64, p, i64, i64, p, p, p]
        lib.oracle_entries_i4.argtypes = [i64, p, i64, p, i64, i64, p, p, p]
        lib.oracle_float_to_half.argtypes = [ctypes.c_float]
        lib.oracle_float_to_half.restype = ctypes.c_uint16
        lib.oracle_dequant.argtypes = [i64, i64, p, i64, p, p, p, i64, i32]
        lib.oracle_dequant.restype = i32
        lib.oracle_dequant_entries.argtypes = [i64, p, p, p, p, i32]
        lib.oracle_dequant_entries.restype = i32
        lib.oracle_gemm_f16_rowb.argtypes = lib.oracle_gemm_f16.argtypes
        lib.oracle_gemm_i8_rowb.argtypes = lib.oracle_gemm_i8.argtypes
        lib.oracle_gemm_i4_rowb.argtypes = lib.oracle_gemm_i4.argtypes
        lib.oracle_entries_f16_rowb.argtypes = lib.oracle_entries_f16.argtypes
        lib.oracle_entries_i8_rowb.argtypes = lib.oracle_entries_i8.argtypes
        lib.oracle_entries_i4_rowb.argtypes = lib.oracle_entries_i4.argtypes
        for f in (lib.oracle_gemm_f16_rowb, lib.oracle_gemm_i8_rowb, lib.oracle_gemm_i4_rowb,
                  lib.oracle_entries_f16_rowb, lib.oracle_entries_i8_rowb,
                  lib.oracle_entries_i4_rowb):
            f.restype = i32
        for f in (lib.oracle_gemm_f16, lib.oracle_gemm_i8, lib.oracle_gemm_i4,
                  lib.oracle_entries_f16, lib.oracle_entries_i8, lib.oracle_entries_i4):
            f.restype = i32
        _lib = lib
    return _lib


def _c(x, dtype):
    a = np.ascontiguousarray(x, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(bits)


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")


def gemm_f16(A, Bt, K=None, threads=None):
    """FP16 product in fp64.  Returns (R, S): R = A*B, S = sum_k |a_ik b_kj|."""
    A, pa = _c(A, np.float16)
    Bt, pb = _c(Bt, np.float16)
    M, N = A.shape[0], Bt.shape[0]
    K = A.shape[1] if K is None else K
    R = np.zeros((M, N), np.float64)
    S = np.zeros((M, N), np.float64)
    _check(_load().oracle_gemm_f16(M, N, K, pa, A.shape[1], pb, Bt.shape[1],
                                   R.ctypes.data_as(ctypes.c_void_p),
                                   S.ctypes.data_as(ctypes.c_void_p), N,
                                   threads or default_threads()))
    return R, S


def gemm_i8(A, Bt, K=None, threads=None):
    """INT8 product, exact, as int64 (M, N)."""
    A, pa = _c(A, np.int8)
    Bt, pb = _c(Bt, np.int8)
    M, N = A.shape[0], Bt.shape[0]
    K = A.shape[1] if K is None else K
    C = np.zeros((M, N), np.int64)
    _check(_load().oracle_gemm_i8(M, N, K, pa, A.shape[1], pb, Bt.shape[1],
                                  C.ctypes.data_as(ctypes.c_void_p), N,
                                  threads or default_threads()))
    return C


def gemm_i4(Ap, Btp, K=None, threads=None):
    """Packed INT4 product (arrays of bytes, two values each), exact, as int64 (M, N)."""
    Ap, pa = _c(Ap, np.uint8)
    Btp, pb = _c(Btp, np.uint8)
    M, N = Ap.shape[0], Btp.shape[0]
    K = 2 * Ap.shape[1] if K is None else K
    C = np.zeros((M, N), np.int64)
    _check(_load().oracle_gemm_i4(M, N, K, pa, 2 * Ap.shape[1], pb, 2 * Btp.shape[1],
                                  C.ctypes.data_as(ctypes.c_void_p), N,
                                  threads or default_threads()))
    return C


def _idx(rows, cols):
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows and cols differ in length")
    return r, c


def entries_f16(A, Bt, rows, cols, K=None):
    """(R, S) at the listed (row, col) positions only."""
    A, pa = _c(A, np.float16)
    Bt, pb = _c(Bt, np.float16)
    r, c = _idx(rows, cols)
    K = A.shape[1] if K is None else K
    R = np.zeros(r.shape, np.float64)
    S = np.zeros(r.shape, np.float64)
    _check(_load().oracle_entries_f16(K, pa, A.shape[1], pb, Bt.shape[1], r.size,
                                      r.ctypes.data_as(ctypes.c_void_p),
                                      c.ctypes.data_as(ctypes.c_void_p),
                                      R.ctypes.data_as(ctypes.c_void_p),
                                      S.ctypes.data_as(ctypes.c_void_p)))
    return R, S


def entries_i8(A, Bt, rows, cols, K=None):
    A, pa = _c(A, np.int8)
    Bt, pb = _c(Bt, np.int8)
    r, c = _idx(rows, cols)
    K = A.shape[1] if K is None else K
    C = np.zeros(r.shape, np.int64)
    _check(_load().oracle_entries_i8(K, pa, A.shape[1], pb, Bt.shape[1], r.size,
                                     r.ctypes.data_as(ctypes.c_void_p),
                                     c.ctypes.data_as(ctypes.c_void_p),
                                     C.ctypes.data_as(ctypes.c_void_p)))
    return C


def entries_i4(Ap, Btp, rows, cols, K=None):
    Ap, pa = _c(Ap, np.uint8)
    Btp, pb = _c(Btp, np.uint8)
    r, c = _idx(rows, cols)
    K = 2 * Ap.shape[1] if K is None else K
    C = np.zeros(r.shape, np.int64)
    _check(_load().oracle_entries_i4(K, pa, 2 * Ap.shape[1], pb, 2 * Btp.shape[1], r.size,
                                     r.ctypes.data_as(ctypes.c_void_p),
                                     c.ctypes.data_as(ctypes.c_void_p),
                                     C.ctypes.data_as(ctypes.c_void_p)))
    return C


def fp16_bound(R, S, rel=1e-3):
    """Per-element tolerance of the FP16 path: rel * S (fp64 summation error is far below)."""
    return rel * S


def float_to_half(x: float) -> int:
    """binary32 value -> binary16 bits (round to nearest even), the oracle's own conversion."""
    return int(_load().oracle_float_to_half(x))


def dequant(S, scale_a, scale_b, half_out=False):
    """C[i][j] = ((float)S[i][j] * scale_a[i]) * scale_b[j] in binary32, optionally rounded to
    binary16.  S is an int64 (M, N) array of exact integer sums.  Returns float32, or float16
    when half_out."""
    S, ps = _c(S, np.int64)
    sa, pa = _c(scale_a, np.float32)
    sb, pb = _c(scale_b, np.float32)
    M, N = S.shape
    if sa.shape != (M,) or sb.shape != (N,):
        raise ValueError("scale_a must hold M values and scale_b N values")
    C = np.zeros((M, N), np.uint16 if half_out else np.float32)
    _check(_load().oracle_dequant(M, N, ps, N, pa, pb, C.ctypes.data_as(ctypes.c_void_p), N,
                                  1 if half_out else 0))
    return C.view(np.float16) if half_out else C


def dequant_entries(S, scale_a, scale_b, half_out=False):
    """Elementwise form of dequant: C[t] = ((float)S[t] * scale_a[t]) * scale_b[t] for
    equal-length 1-D arrays (the row and column scale of each listed entry)."""
    S, ps = _c(S, np.int64)
    sa, pa = _c(scale_a, np.float32)
    sb, pb = _c(scale_b, np.float32)
    if S.ndim != 1 or sa.shape != S.shape or sb.shape != S.shape:
        raise ValueError("S, scale_a and scale_b must be 1-D and of equal length")
    C = np.zeros(S.shape, np.uint16 if half_out else np.float32)
    _check(_load().oracle_dequant_entries(S.size, ps, pa, pb, C.ctypes.data_as(ctypes.c_void_p),
                                          1 if half_out else 0))
    return C.view(np.float16) if half_out else C


# ---------------------------------------------------------------------------
# B row-major: B is a (K, ldb) array (int4: (K, ldb/2) bytes packed along N)

def _rowb_dims(A, B, N, K, packed):
    width = 2 * B.shape[1] if packed else B.shape[1]
    N = width if N is None else N
    K = (2 * A.shape[1] if packed else A.shape[1]) if K is None else K
    if N > width or K > B.shape[0]:
        raise ValueError("B holds fewer than K rows or N columns")
    return N, K, width


def gemm_f16_rowb(A, B, N=None, K=None, threads=None):
    """FP16 product with B row-major, in fp64: returns (R, S) as gemm_f16."""
    A, pa = _c(A, np.float16)
    B, pb = _c(B, np.float16)
    N, K, ldb = _rowb_dims(A, B, N, K, False)
    M = A.shape[0]
    R = np.zeros((M, N), np.float64)
    S = np.zeros((M, N), np.float64)
    _check(_load().oracle_gemm_f16_rowb(M, N, K, pa, A.shape[1], pb, ldb,
                                        R.ctypes.data_as(ctypes.c_void_p),
                                        S.ctypes.data_as(ctypes.c_void_p), N,
                                        threads or default_threads()))
    return R, S


def gemm_i8_rowb(A, B, N=None, K=None, threads=None):
    """INT8 product with B row-major, exact, as int64 (M, N)."""
    A, pa = _c(A, np.int8)
    B, pb = _c(B, np.int8)
    N, K, ldb = _rowb_dims(A, B, N, K, False)
    C = np.zeros((A.shape[0], N), np.int64)
    _check(_load().oracle_gemm_i8_rowb(A.shape[0], N, K, pa, A.shape[1], pb, ldb,
                                       C.ctypes.data_as(ctypes.c_void_p), N,
                                       threads or default_threads()))
    return C


def gemm_i4_rowb(Ap, Bp, N=None, K=None, threads=None):
    """Packed INT4 product with B row-major (packed along N), exact, as int64 (M, N)."""
    Ap, pa = _c(Ap, np.uint8)
    Bp, pb = _c(Bp, np.uint8)
    N, K, ldb = _rowb_dims(Ap, Bp, N, K, True)
    C = np.zeros((Ap.shape[0], N), np.int64)
    _check(_load().oracle_gemm_i4_rowb(Ap.shape[0], N, K, pa, 2 * Ap.shape[1], pb, ldb,
                                       C.ctypes.data_as(ctypes.c_void_p), N,
                                       threads or default_threads()))
    return C


def entries_f16_rowb(A, B, rows, cols, K=None):
    A, pa = _c(A, np.float16)
    B, pb = _c(B, np.float16)
    r, c = _idx(rows, cols)
    K = A.shape[1] if K is None else K
    R = np.zeros(r.shape, np.float64)
    S = np.zeros(r.shape, np.float64)
    _check(_load().oracle_entries_f16_rowb(K, pa, A.shape[1], pb, B.shape[1], r.size,
                                           r.ctypes.data_as(ctypes.c_void_p),
                                           c.ctypes.data_as(ctypes.c_void_p),
                                           R.ctypes.data_as(ctypes.c_void_p),
                                           S.ctypes.data_as(ctypes.c_void_p)))
    return R, S


def entries_i8_rowb(A, B, rows, cols, K=None):
    A, pa = _c(A, np.int8)
    B, pb = _c(B, np.int8)
    r, c = _idx(rows, cols)
    K = A.shape[1] if K is None else K
    C = np.zeros(r.shape, np.int64)
    _check(_load().oracle_entries_i8_rowb(K, pa, A.shape[1], pb, B.shape[1], r.size,
                                          r.ctypes.data_as(ctypes.c_void_p),
                                          c.ctypes.data_as(ctypes.c_void_p),
                                          C.ctypes.data_as(ctypes.c_void_p)))
    return C


def entries_i4_rowb(Ap, Bp, rows, cols, K=None):
    Ap, pa = _c(Ap, np.uint8)
    Bp, pb = _c(Bp, np.uint8)
    r, c = _idx(rows, cols)
    K = 2 * Ap.shape[1] if K is None else K
    C = np.zeros(r.shape, np.int64)
    _check(_load().oracle_entries_i4_rowb(K, pa, 2 * Ap.shape[1], pb, 2 * Bp.shape[1], r.size,
                                          r.ctypes.data_as(ctypes.c_void_p),
                                          c.ctypes.data_as(ctypes.c_void_p),
                                          C.ctypes.data_as(ctypes.c_void_p)))
    return C
