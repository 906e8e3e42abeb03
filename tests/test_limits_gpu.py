"""GPU cases at the limits the header states.

* The largest K whose int32 sums cannot overflow: INT8 K = 131071 and INT4
  K = 131070 (the largest even K; the INT4 planes sum 256 * a * b, so the
  scaled sum of all -8 products, 16384 * 131070, sits just below 2^31).
  Checked against the closed forms at the extreme values, on the plain, the
  K-split and the row-major-B kernels; FP16 with all-ones operands at
  K = 131072 (every partial sum an integer below 2^24, so C = K exactly).
* The largest leading dimensions: rows of 4 MiB for A, B and C, so that a
  256-row tile spans 1 GiB of offsets, checked against the oracle on ragged
  M, N and K; and rows of 4 MiB for a row-major B on the K-split tiles, whose
  stages span up to 1024 rows of B.

Operands' padding past K holds poison, and every case prints its name before
it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_ROW_BYTES = 1 << 22


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def filled(rows, ld, cols, value, poison, dtype, dev):
    """(rows, ld) device buffer: `value` in the first `cols` columns, `poison` after."""
    t = torch.full((rows, ld), poison, dtype=dtype, device=dev)
    t[:, :cols] = value
    return t[:, :cols]


# (M, N): the K-split 32 x 32 tile at M = 16, the plain tiles at M = 130
SHAPES = [(16, 96), (130, 96)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("b_value,expect", [(-128, 16384), (127, -16256)])
def test_int8_largest_k(pd, dev, M, N, b_value, expect):
    K, ld = 131071, 131072
    gu.note(f"[case] i8 largest K={K} M={M} N={N} b={b_value}")
    A = filled(M, ld, K, -128, 127, torch.int8, dev)
    Bt = filled(N, ld, K, b_value, 127, torch.int8, dev)
    C = pd.gemm_i8(A, Bt)
    B = filled(K, N + 16, N, b_value, 127, torch.int8, dev)   # the same B, row-major
    Cr = pd.gemm_i8_rowb(A, B)
    torch.cuda.synchronize()
    assert expect * K < 2 ** 31
    assert torch.all(C == expect * K) and torch.all(Cr == expect * K)


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("b_byte,expect", [(0x88, 64), (0x77, -56)])
def test_int4_largest_k(pd, dev, M, N, b_byte, expect):
    K, ld_bytes = 131070, 65536          # K / 2 = 65535 bytes of data per row
    gu.note(f"[case] i4 largest K={K} M={M} N={N} b=0x{b_byte:02x}")
    A = filled(M, ld_bytes, K // 2, 0x88, 0x77, torch.uint8, dev)     # all -8
    Bt = filled(N, ld_bytes, K // 2, b_byte, 0x77, torch.uint8, dev)
    C = pd.gemm_i4(A, Bt, K)
    B = filled(K, N // 2 + 16, N // 2, b_byte, 0x77, torch.uint8, dev)   # row-major, packed along N
    Cr = pd.gemm_i4_rowb(A, B, K, N)
    torch.cuda.synchronize()
    assert 16384 * K < 2 ** 31   # the scaled sum of the all -8 case
    assert torch.all(C == expect * K) and torch.all(Cr == expect * K)


@pytest.mark.parametrize("M,N", SHAPES)
def test_f16_long_k_ones(pd, dev, M, N):
    K = 131072
    gu.note(f"[case] f16 ones K={K} M={M} N={N}")
    A = filled(M, K + 64, K, 1.0, float("nan"), torch.float16, dev)
    Bt = filled(N, K + 64, K, 1.0, float("nan"), torch.float16, dev)
    C = pd.gemm_f16(A, Bt)
    torch.cuda.synchronize()
    assert torch.all(C == K)


LD = {"f16": MAX_ROW_BYTES // 2, "i8": MAX_ROW_BYTES, "i4": MAX_ROW_BYTES * 2}   # in elements


# (tile configuration, ranges of K split across workgroups): the 64 x 64 and
# 128 x 64 tiles split two (FP16) or three ways start each range's A and B
# at an offset of whole stages into rows of 4 MiB
SPLITS = {"f16": 2, "i8": 3, "i4": 3}


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("cfg,split", [(0, False), (4, False), (10, False), (3, False), (9, False), (2, True),
                                       (5, True)])
def test_largest_leading_dimensions(pd, dev, prec, cfg, split):
    # 256 x 256 and 256 x 128 tiles (configurations 0 and 4, FP16 and INT8 on 16 x 16 MFMAs;
    # 10: 0 on 32 x 32 ones), the K-split 32 x 32 and 64 x 64 tiles (3, 9), and K split
    # across workgroups (2, 5), with rows of A, B and C of 4 MiB; M, N and K ragged
    M, N, K = 250, 70, 200 if not split else 1000
    splits = SPLITS[prec] if split else None
    ld = LD[prec]
    ldc = MAX_ROW_BYTES // 4
    gu.note(f"[case] largest ld {prec} cfg={cfg} splits={splits} lda=ldb={ld} ldc={ldc}")
    A, Bt = synth.operands(prec, M, N, K, 77, 78)
    cols = K // 2 if prec == "i4" else K
    ld_cols = ld // 2 if prec == "i4" else ld
    dt = {"f16": torch.float16, "i8": torch.int8, "i4": torch.uint8}[prec]
    poison = {"f16": float("nan"), "i8": 127, "i4": 0x77}[prec]
    Ad = torch.full((M, ld_cols), poison, dtype=dt, device=dev)
    Ad[:, :cols] = torch.from_numpy(A).to(dev)
    Bd = torch.full((N, ld_cols), poison, dtype=dt, device=dev)
    Bd[:, :cols] = torch.from_numpy(Bt).to(dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    Cbuf = torch.zeros((M, ldc), dtype=out_dtype, device=dev)
    out = Cbuf[:, :N]
    if prec == "f16":
        pd.gemm_f16(Ad[:, :cols], Bd[:, :cols], out=out, cfg=cfg, splits=splits)
    elif prec == "i8":
        pd.gemm_i8(Ad[:, :cols], Bd[:, :cols], out=out, cfg=cfg, splits=splits)
    else:
        pd.gemm_i4(Ad[:, :cols], Bd[:, :cols], K, out=out, cfg=cfg, splits=splits)
    torch.cuda.synchronize()
    C = out.cpu().numpy()
    assert torch.count_nonzero(Cbuf[:, N:]) == 0, "stores past column N"
    del Ad, Bd, Cbuf
    if prec == "f16":
        R, S = oracle.gemm_f16(A, Bt)
        gu.assert_f16_close(C, R, S, f"largest ld {prec} cfg{cfg}")
    else:
        ref = oracle.gemm_i8(A, Bt) if prec == "i8" else oracle.gemm_i4(A, Bt, K)
        gu.assert_int_equal(C, ref, f"largest ld {prec} cfg{cfg}")


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("cfg,split", [(0, False), (4, False), (10, False), (3, False), (6, False), (9, False),
                                       (2, True), (5, True)])
def test_largest_leading_dimension_row_major_b(pd, dev, prec, cfg, split):
    # B row-major with rows of 4 MiB, on the 256 x 256 and 256 x 128 tiles (0, 4; 10: 0 on
    # 32 x 32 MFMAs) and on the K-split
    # tiles (3: 32 x 32, 6: 64 x 32, 9: 64 x 64), whose waves each stage their own slice of
    # rows of B; K reaches the last slice of a stage (a 64 x 32 INT4 stage spans
    # 1024 rows of B, 4 GiB at this row size)
    # (2, 5: K split across workgroups, each range's B starting whole stages of
    # 4 MiB rows in)
    M, N, K = 50, 70, 1000
    splits = SPLITS[prec] if split else None
    ld = LD[prec]
    ldc = MAX_ROW_BYTES // 4
    gu.note(f"[case] largest ldb row-major B {prec} cfg={cfg} splits={splits} ldb={ld} ldc={ldc} K={K}")
    if prec == "i4":
        A = synth.pack_int4(synth.int4_values(M, K, 91))
        B = synth.pack_int4(np.ascontiguousarray(synth.int4_values(N, K, 92).T))   # (K, N/2)
        cols_a, cols_b, ld_cols = K // 2, N // 2, ld // 2
    else:
        A, Bt = synth.operands(prec, M, N, K, 91, 92)
        B = np.ascontiguousarray(Bt.T)                                           # (K, N)
        cols_a, cols_b, ld_cols = K, N, ld
    dt = {"f16": torch.float16, "i8": torch.int8, "i4": torch.uint8}[prec]
    poison = {"f16": float("nan"), "i8": 127, "i4": 0x77}[prec]
    Ad = torch.full((M, gu.round_up(cols_a, 16) + 16), poison, dtype=dt, device=dev)
    Ad[:, :cols_a] = torch.from_numpy(A).to(dev)
    # two extra rows past K, all poison
    Bd = torch.full((K + 2, ld_cols), poison, dtype=dt, device=dev)
    Bd[:K, :cols_b] = torch.from_numpy(B).to(dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    Cbuf = torch.zeros((M, ldc), dtype=out_dtype, device=dev)
    out = Cbuf[:, :N]
    Bv = Bd[:K, :cols_b]
    if prec == "f16":
        pd.gemm_f16_rowb(Ad[:, :cols_a], Bv, out=out, cfg=cfg, splits=splits)
    elif prec == "i8":
        pd.gemm_i8_rowb(Ad[:, :cols_a], Bv, out=out, cfg=cfg, splits=splits)
    else:
        pd.gemm_i4_rowb(Ad[:, :cols_a], Bv, K, N, out=out, cfg=cfg, splits=splits)
    torch.cuda.synchronize()
    C = out.cpu().numpy()
    assert torch.count_nonzero(Cbuf[:, N:]) == 0, "stores past column N"
    del Ad, Bd, Bv, Cbuf
    if prec == "f16":
        R, S = oracle.gemm_f16_rowb(A, B, N=N, K=K)
        gu.assert_f16_close(C, R, S, f"largest ldb rowb {prec} cfg{cfg}")
    else:
        ref = (oracle.gemm_i8_rowb if prec == "i8" else oracle.gemm_i4_rowb)(A, B, N=N, K=K)
        gu.assert_int_equal(C, ref, f"largest ldb rowb {prec} cfg{cfg}")
