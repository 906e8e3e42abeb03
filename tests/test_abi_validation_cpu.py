"""Property test of the C ABI's argument checks: random argument sets against an
independent model of the rules include/pdgemm.h states, in the order the
library applies them.  Only argument sets the model rejects are passed to the
library (they return before any HIP call), so no GPU is needed."""
from __future__ import annotations

import ctypes
import os

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "precision_dense_gemm_amd", "libpdgemm.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpdgemm.so not built")

OK, EDIM, ELD, ENULL, EI4, EALIGN, ECFG = 0, -1, -2, -3, -4, -5, -6
BITS = {0: 16, 1: 8, 2: 4}
MAX_ROW = 1 << 22


def model(prec, cfg, epi, rowb, M, N, K, A, lda, B, ldb, C, ldc, sa, sb, ksplit_cfgs, ncfg, tiles=None):
    """Expected return code, or None when the call would reach the GPU.  tiles maps a
    configuration to (block rows, block cols, threads) for the work-item limit."""
    if not (0 <= prec <= 2) or not (0 <= cfg < ncfg):
        return ECFG
    if epi and prec == 0:
        return ECFG
    if M < 0 or N < 0 or K < 0 or M > 2 ** 31 - 1 or N > 2 ** 31 - 1 or K > 2 ** 30:
        return EDIM
    if prec == 2 and K > 131071:
        return EDIM
    if lda < K or ldb < (N if rowb else K) or ldc < N:
        return ELD
    if prec == 2 and (K % 2 or lda % 2 or ldb % 2):
        return EI4
    if M == 0 or N == 0:
        return OK
    if not C or (K > 0 and (not A or not B)):
        return ENULL
    if epi and (not sa or not sb):
        return ENULL
    csize = 2 if epi == 2 else 4
    if lda > MAX_ROW * 8 // BITS[prec] or ldb > MAX_ROW * 8 // BITS[prec] or ldc > MAX_ROW // csize:
        return ELD
    if (lda * BITS[prec] // 8) % 16 or (ldb * BITS[prec] // 8) % 16:
        return EALIGN
    if A % 16 or B % 16 or C % csize:
        return EALIGN
    if epi and (sa % 4 or sb % 4):
        return EALIGN
    if tiles is not None:
        bm, bn, threads = tiles[cfg]
        if -(-M // bm) * -(-N // bn) * threads > 2 ** 32 - 1:
            return EDIM
    return None


@pytest.fixture(scope="module")
def lib():
    # loaded here, never at import: collection imports this module in GPU runs too, and a
    # HIP library opened there, before torch set up the device, left every later GPU call
    # of the process failing (hipErrorNoDevice)
    L = ctypes.CDLL(LIB)
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.pdgemm_gemm_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.pdgemm_gemm_rowb_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.pdgemm_dequant_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p]
    L.pdgemm_config_info.argtypes = [i] + [ctypes.POINTER(i)] * 5
    n = L.pdgemm_num_configs()
    ks, tiles = set(), {}
    for c in range(n):
        v = [ctypes.c_int() for _ in range(5)]
        L.pdgemm_config_info(c, *[ctypes.byref(x) for x in v])
        bm, bn, wm, wn, th = (x.value for x in v)
        tiles[c] = (bm, bn, th)
        if th > (bm // wm) * (bn // wn) * 64:
            ks.add(c)
    return L, n, ks, tiles


def weighted(common, rare, pct_rare):
    """`rare` in about pct_rare percent of the draws, else `common`."""
    return st.integers(0, 99).flatmap(lambda r: rare if r < pct_rare else common)


# mostly plausible values, with the boundary and invalid ones mixed in
dims = weighted(st.integers(1, 300), st.one_of(st.integers(-3, 0), st.sampled_from(
    [2 ** 30, 2 ** 30 + 1, 131071, 131072, 2 ** 31])), 12)
lds = weighted(st.integers(1, 20).map(lambda x: 32 * x), st.one_of(st.integers(-2, 600), st.sampled_from(
    [2 ** 21, 2 ** 22, 2 ** 22 + 32, 2 ** 23 + 32, 2 ** 61, 2 ** 62])), 15)
ptrs = weighted(st.sampled_from([0x10000, 0x20000, 0x30000]), st.one_of(st.just(0), st.sampled_from(
    [0x10000, 0x20000]).flatmap(lambda b: st.integers(1, 17).map(lambda o: b + o))), 10)

def combos(ncfg):
    """(precision, configuration, epilogue, row-major B): valid ones, and in about one draw
    in ten an invalid precision or configuration."""
    valid = [(p, c, e, r) for p in range(3) for c in range(ncfg) for e in range(3) for r in (False, True)
             if not (e and p == 0) and not (e and r)]
    invalid = [(p, c, e, False) for p in (-1, 0, 1, 3) for c in (-1, 0, ncfg, ncfg + 1) for e in (0, 1)]
    return weighted(st.sampled_from(valid), st.sampled_from(invalid), 10)


@settings(max_examples=4000, deadline=None)
@given(data=st.data(), M=dims, N=dims, K=dims, A=ptrs, lda=lds, B=ptrs, ldb=lds, C=ptrs, ldc=lds,
       sa=ptrs, sb=ptrs)
def test_argument_checks_follow_the_documented_rules(lib, data, M, N, K, A, lda, B, ldb, C, ldc,
                                                     sa, sb):
    L, ncfg, ks, tiles = lib
    prec, cfg, epi, rowb = data.draw(combos(ncfg))
    want = model(prec, cfg, epi, rowb, M, N, K, A, lda, B, ldb, C, ldc, sa, sb, ks, ncfg, tiles)
    if want is None:
        return   # a valid call: it would launch on the GPU
    if epi:
        got = L.pdgemm_dequant_cfg(prec, cfg, M, N, K, A or None, lda, B or None, ldb, sa or None,
                                   sb or None, C or None, ldc, 1 if epi == 2 else 0, None)
    elif rowb:
        got = L.pdgemm_gemm_rowb_cfg(prec, cfg, M, N, K, A or None, lda, B or None, ldb, C or None,
                                     ldc, None)
    else:
        got = L.pdgemm_gemm_cfg(prec, cfg, M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                None)
    assert got == want, (prec, cfg, epi, rowb, M, N, K, A, lda, B, ldb, C, ldc, sa, sb)
