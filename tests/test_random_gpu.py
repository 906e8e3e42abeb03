"""Seeded random parity sweep on the GPU: for every precision and entry-point family
(plain, row-major B, dequantizing to fp32 or binary16, and the plain and row-major
GEMMs with K split across workgroups), shapes, padded leading dimensions and a tile
configuration (the entry points' own choice or any of them; for the split families a
split tile and 1-8 ranges, 1-2 for FP16) are drawn from a fixed seed, and every output is compared in full with the oracle (integers
and dequantized outputs bit for bit, FP16 within 1e-3 * sum |a*b|).  Operands sit in
poison-padded buffers and outputs in sentinel-guarded ones."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = 60   # per (precision, family)


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def draw(rng, prec, ncfg):
    M = int(rng.choice([rng.integers(1, 40), rng.integers(1, 300), rng.integers(200, 700)]))
    N = int(rng.choice([rng.integers(1, 40), rng.integers(1, 300), rng.integers(200, 900)]))
    K = int(rng.choice([rng.integers(1, 70), rng.integers(1, 600), rng.integers(500, 1500)]))
    if prec == "i4":
        K += K % 2
    cfg = None if rng.random() < 0.4 else int(rng.integers(0, ncfg))
    pad = int(rng.integers(0, 3))
    return M, N, K, cfg, pad


def padded(host, width, fill, dev):
    return gu.to_device_padded(torch, host, width, fill, dev)


FAMILIES = ["plain", "rowb", "dequant32", "dequant16", "split", "split_rowb"]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
def test_random_shapes(pd, dev, prec, family):
    if family.startswith("dequant") and prec == "f16":
        pytest.skip("the dequantizing epilogue is for the integer paths")
    rng = np.random.default_rng({"f16": 1, "i8": 2, "i4": 3}[prec] * 100 + FAMILIES.index(family))
    poison = gu.POISON[prec]
    base = {"split": "plain", "split_rowb": "rowb"}.get(family, family)
    for case in range(CASES):
        M, N, K, cfg, pad = draw(rng, prec, pd.num_configs())
        splits = None
        if family.startswith("split"):
            cfg = int(rng.choice([2, 5]))
            splits = int(rng.integers(1, 3 if prec == "f16" else 9))
        seed = int(rng.integers(0, 2 ** 31))
        gu.note(f"[case] random {prec} {family} #{case}: M={M} N={N} K={K} cfg={cfg} splits={splits} "
                f"pad={pad} seed={seed}")
        A, Bt = synth.operands(prec, M, N, K, seed, seed + 1)
        a_w = gu.round_up(A.shape[1], 16 // (2 if prec == "f16" else 1)) + pad * 16 // (2 if prec == "f16" else 1)
        Ad = padded(A, max(a_w, 16 // (2 if prec == "f16" else 1)), poison, dev)
        odt = {"plain": torch.float32 if prec == "f16" else torch.int32, "rowb": torch.float32 if prec == "f16"
               else torch.int32, "dequant32": torch.float32, "dequant16": torch.float16}[base]
        ldc = N + int(rng.integers(0, 5))
        if odt == torch.float16:
            buf = torch.full((M + 2, ldc), 0x7DAD, dtype=torch.int16, device=dev).view(torch.float16)
        else:
            buf = torch.empty((M + 2, ldc), dtype=torch.int32, device=dev).fill_(gu.C_SENTINEL_BITS).view(odt)
        out = buf[:M, :N]
        if base == "rowb":
            if prec == "i4":
                vals = synth.unpack_int4(Bt)[:, :K].T        # (K, N)
                if N % 2:
                    vals = np.hstack([vals, np.zeros((K, 1), np.int8)])
                B = synth.pack_int4(np.ascontiguousarray(vals))
            else:
                B = np.ascontiguousarray(Bt.T)
            b_w = gu.round_up(B.shape[1], 16 // (2 if prec == "f16" else 1)) + pad * 16 // (2 if prec == "f16" else 1)
            Bbuf = np.full((K + 1, max(b_w, 16)), poison, dtype=B.dtype)
            Bbuf[:K, :B.shape[1]] = B
            Bd = torch.from_numpy(Bbuf).to(dev)[:K, :B.shape[1]]
            if prec == "f16":
                pd.gemm_f16_rowb(Ad, Bd, out=out, cfg=cfg, splits=splits)
                R, S = oracle.gemm_f16_rowb(A, B, N=N, K=K)
            elif prec == "i8":
                pd.gemm_i8_rowb(Ad, Bd, out=out, cfg=cfg, splits=splits)
                ref = oracle.gemm_i8_rowb(A, B, N=N, K=K)
            else:
                pd.gemm_i4_rowb(Ad, Bd, K, N, out=out, cfg=cfg, splits=splits)
                ref = oracle.gemm_i4_rowb(A, B, N=N, K=K)
        else:
            b_w = gu.round_up(Bt.shape[1], 16 // (2 if prec == "f16" else 1)) + pad * 16 // (2 if prec == "f16" else 1)
            Bd = padded(Bt, max(b_w, 16 // (2 if prec == "f16" else 1)), poison, dev)
            if base == "plain":
                if prec == "f16":
                    pd.gemm_f16(Ad, Bd, out=out, cfg=cfg, splits=splits)
                    R, S = oracle.gemm_f16(A, Bt, K=K)
                elif prec == "i8":
                    pd.gemm_i8(Ad, Bd, out=out, cfg=cfg, splits=splits)
                    ref = oracle.gemm_i8(A, Bt, K=K)
                else:
                    pd.gemm_i4(Ad, Bd, K, out=out, cfg=cfg, splits=splits)
                    ref = oracle.gemm_i4(A, Bt, K=K)
            else:
                sa, sb = synth.f32_scales(M, seed + 2), synth.f32_scales(N, seed + 3)
                sad, sbd = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
                if prec == "i8":
                    pd.gemm_i8_dequant(Ad, Bd, sad, sbd, out=out, cfg=cfg)
                    Sx = oracle.gemm_i8(A, Bt, K=K)
                else:
                    pd.gemm_i4_dequant(Ad, Bd, sad, sbd, K, out=out, cfg=cfg)
                    Sx = oracle.gemm_i4(A, Bt, K=K)
                want = oracle.dequant(Sx, sa, sb, half_out=(family == "dequant16"))
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        bits = host.view(np.int16 if odt == torch.float16 else np.int32)
        outside = np.ones(bits.shape, dtype=bool)
        outside[:M, :N] = False
        sentinel = np.int16(0x7DAD) if odt == torch.float16 else np.int32(gu.C_SENTINEL_BITS)
        assert np.all(bits[outside] == sentinel), f"stores outside M x N in case #{case}"
        C = host[:M, :N]
        what = f"{prec} {family} #{case} M={M} N={N} K={K} cfg={cfg} splits={splits}"
        if family.startswith("dequant"):
            gw = want.view(np.uint16 if family == "dequant16" else np.uint32)
            gc = C.view(np.uint16 if family == "dequant16" else np.uint32)
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(C), nan) and np.array_equal(gc[~nan], gw[~nan]), what
        elif prec == "f16":
            gu.assert_f16_close(C, R, S, what)
        else:
            gu.assert_int_equal(C, ref, what)
