"""GPU parity of the GEMM with B row-major (element (k, j) at B[k*ldb + j];
INT4 packed two per byte along N) against the CPU oracle's row-major form.

Integers bit-exact; FP16 within 1e-3 * sum |a*b|.  B sits in a buffer whose
rows are wider than N and which has two extra rows past K, all padding holding
poison (NaN / 127 / 0x77), so a read outside the K x N extent that reached a
result would show; C sits in a sentinel-filled guard buffer.  At full size the
row-major result must also equal the column-major kernel's on the same matrix,
bit for bit (the same products in the same order).  Every case prints its name
before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PRECS = ("f16", "i8", "i4")


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def rowb_operands(prec, M, N, K, seed):
    """A (M x K, packed along K for i4) and row-major B (K x N, packed along N for i4),
    drawn as the column-major operands of the same seeds and laid out row-major."""
    if prec == "i4":
        A = synth.pack_int4(synth.int4_values(M, K, seed))
        Bvals = synth.int4_values(N, K, seed + 1).T          # (K, N)
        if N % 2:   # packing along N needs an even width; the extra column is outside N
            Bvals = np.hstack([Bvals, np.zeros((K, 1), np.int8)])
        return A, synth.pack_int4(np.ascontiguousarray(Bvals)), Bvals[:, :N]
    A, Bt = synth.operands(prec, M, N, K, seed, seed + 1)
    return A, np.ascontiguousarray(Bt.T), None


def oracle_rowb(prec, A, B, N, K):
    if prec == "f16":
        return oracle.gemm_f16_rowb(A, B, N=N, K=K)
    if prec == "i8":
        return oracle.gemm_i8_rowb(A, B, N=N, K=K)
    return oracle.gemm_i4_rowb(A, B, N=N, K=K)


def check(prec, C, ref, what):
    if prec == "f16":
        gu.assert_f16_close(C, ref[0], ref[1], what)
    else:
        gu.assert_int_equal(C, ref, what)


def run_case(pd, dev, prec, M, N, K, seed, cfg=None):
    gu.note(f"[case] rowb {prec} M={M} N={N} K={K} seed={seed} cfg={cfg}")
    A, B, _ = rowb_operands(prec, M, N, K, seed)
    poison = gu.POISON[prec]
    if prec == "i4":
        Ad = gu.to_device_padded(torch, A, gu.round_up(K // 2, 16) + 16, poison, dev)
        nb = B.shape[1]                                    # bytes of N per row
        ldb_b = gu.round_up(nb, 16) + 16
    else:
        align = gu.ld_align(prec)
        Ad = gu.to_device_padded(torch, A, gu.round_up(K, align) + align, poison, dev)
        nb = N
        ldb_b = gu.round_up(N, align) + align
    Bbuf = np.full((K + 2, ldb_b), poison, dtype=B.dtype)
    Bbuf[:K, :nb] = B
    if prec == "i4" and N % 2:
        # odd N: the high nibble of each row's last byte lies outside; poison it
        Bbuf[:K, nb - 1] = (Bbuf[:K, nb - 1] & 0x0F) | 0x70
    Bd = torch.from_numpy(Bbuf).to(dev)[:K, :nb]
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    buf, out = gu.guarded_out(torch, M, N, gu.round_up(N, 4) + 4, out_dtype, dev)
    if prec == "f16":
        pd.gemm_f16_rowb(Ad, Bd, out=out, cfg=cfg)
    elif prec == "i8":
        pd.gemm_i8_rowb(Ad, Bd, out=out, cfg=cfg)
    else:
        pd.gemm_i4_rowb(Ad, Bd, K, N, out=out, cfg=cfg)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    return A, Bbuf[:K, :nb], out.cpu().numpy()


SMALL = [(1, 1, 2), (2, 3, 8), (16, 8, 16), (31, 33, 18), (65, 63, 130), (127, 129, 128),
         (96, 80, 200), (255, 257, 258), (300, 17, 1000), (17, 300, 1002), (64, 64, 64)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("shape", SMALL, ids=[f"{m}x{n}x{k}" for m, n, k in SMALL])
def test_small_shapes(pd, dev, prec, shape):
    M, N, K = shape
    A, B, C = run_case(pd, dev, prec, M, N, K, 2000 + 7 * M + 13 * N + K)
    check(prec, C, oracle_rowb(prec, A, B, N, K), f"rowb {prec} {shape}")


CFG_SHAPES = [(520, 600, 520), (300, 260, 1030), (64, 700, 130)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
@pytest.mark.parametrize("shape", CFG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in CFG_SHAPES])
def test_every_config(pd, dev, prec, cfg, shape):
    M, N, K = shape
    A, B, C = run_case(pd, dev, prec, M, N, K, 300 + cfg, cfg=cfg)
    check(prec, C, oracle_rowb(prec, A, B, N, K), f"rowb {prec} cfg{cfg} {shape}")


# small M: the K-split tiles (3 = 32 x 32, 6 = 64 x 32), each wave on its own
# slice of K rows of B
KSPLIT = [((16, 700, 1030), 3), ((1, 96, 258), 3), ((50, 8200, 260), 6), ((64, 8192, 130), 6)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("shape,cfg", KSPLIT, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in KSPLIT])
def test_small_m_ksplit(pd, dev, prec, shape, cfg):
    M, N, K = shape
    assert pd.pick_config({"f16": 0, "i8": 1, "i4": 2}[prec], M, N, K) == cfg
    A, B, C = run_case(pd, dev, prec, M, N, K, 900 + M)
    check(prec, C, oracle_rowb(prec, A, B, N, K), f"rowb {prec} small M {shape}")


def test_mma_lab_example_with_row_major_b(pd, dev):
    """The PTX tutorial's 16x8x16 example, with B in its natural row-major form:
    A = I and B[r][c] = 8r + c + 1 give C = B (C[1][2] = 11, C[9][3] = 76)."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mma_lab_identity.json")))
    M, N, K = g["M"], g["N"], g["K"]
    gu.note("[case] rowb mma-lab example")
    B = np.array([[8 * r + c + 1 for c in range(N)] for r in range(K)], dtype=np.float16)
    C = pd.gemm_f16_rowb(torch.from_numpy(np.eye(M, K, dtype=np.float16)).to(dev),
                         torch.from_numpy(B).to(dev)).cpu().numpy()
    for r, c, v in g["printed_entries"]:
        assert C[r, c] == v
    assert np.array_equal(C, B.astype(np.float32))


@pytest.mark.parametrize("K", [64, 2048])
def test_closed_form_extremes(pd, dev, K):
    M, N = 130, 96
    gu.note(f"[case] rowb extremes K={K}")
    C = pd.gemm_i8_rowb(torch.full((M, K), -128, dtype=torch.int8, device=dev),
                        torch.full((K, N), 127, dtype=torch.int8, device=dev)).cpu().numpy()
    assert np.all(C == -16256 * K)
    a = torch.from_numpy(synth.pack_int4(np.full((M, K), -8, np.int8))).to(dev)
    b = torch.from_numpy(synth.pack_int4(np.full((K, N), 7, np.int8))).to(dev)
    assert np.all(pd.gemm_i4_rowb(a, b, K, N).cpu().numpy() == -56 * K)
    C = pd.gemm_f16_rowb(torch.ones((M, K), dtype=torch.float16, device=dev),
                         torch.ones((K, N), dtype=torch.float16, device=dev)).cpu().numpy()
    assert np.all(C == K)


@pytest.mark.parametrize("prec", PRECS)
def test_k_zero(pd, dev, prec):
    M, N = 70, 96
    gu.note(f"[case] rowb {prec} K=0")
    dt = {"f16": torch.float16, "i8": torch.int8, "i4": torch.uint8}[prec]
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    buf, out = gu.guarded_out(torch, M, N, 100, out_dtype, dev)
    A = torch.zeros((M, 16), dtype=dt, device=dev)[:, :0]
    B = torch.zeros((1, N), dtype=dt, device=dev)[:0]
    if prec == "f16":
        pd.gemm_f16_rowb(A, B, out=out)
    elif prec == "i8":
        pd.gemm_i8_rowb(A, B, out=out)
    else:
        pd.gemm_i4_rowb(A, torch.zeros((1, N // 2), dtype=dt, device=dev)[:0], 0, N, out=out)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    assert np.all(out.cpu().numpy() == 0)


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("n", [2048, 8192])
def test_full_size_matches_column_major(pd, dev, prec, n):
    """The workload shapes with B row-major: every element against the oracle, sampled
    entries against its triple loop, and bit equality with the column-major kernel."""
    seed_a = synth.config_seed(6, n, synth.OPERAND_A)
    gu.note(f"[case] rowb {prec} {n}^3 seed {seed_a:#x}")
    A, B, Bvals = rowb_operands(prec, n, n, n, seed_a)
    Bt = synth.pack_int4(np.ascontiguousarray(Bvals.T)) if prec == "i4" else np.ascontiguousarray(B.T)
    Ad, Bd, Btd = (torch.from_numpy(x).to(dev) for x in (A, B, Bt))
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    Cr = torch.empty((n, n), dtype=out_dtype, device=dev)
    Cc = torch.empty((n, n), dtype=out_dtype, device=dev)
    pd.prepare(prec, Ad, Bd, Cr, K=n, rowb=True)      # the launch the benchmark times
    pd.prepare(prec, Ad, Btd, Cc, K=n)
    torch.cuda.synchronize()
    assert torch.equal(Cr.view(torch.int32), Cc.view(torch.int32)), "row-major B differs from column-major B"
    C = Cr.cpu().numpy()
    del Ad, Bd, Btd, Cr, Cc
    gu.check_whole(prec, A, B, n, C, f"rowb {prec} {n}", rowb=True)
    rows, cols = gu.sample_positions(n, n, 512, seed=n + 7)
    got = C[rows, cols]
    if prec == "f16":
        R, S = oracle.entries_f16_rowb(A, B, rows, cols)
        gu.assert_f16_close(got, R, S, f"rowb {prec} {n}")
    else:
        ref = (oracle.entries_i8_rowb if prec == "i8" else oracle.entries_i4_rowb)(A, B, rows, cols)
        gu.assert_int_equal(got, ref, f"rowb {prec} {n}")
