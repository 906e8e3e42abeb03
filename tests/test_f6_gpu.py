"""GPU parity of INT4 on the FP6 matrix cores (the workspace entry points and
the explicit FP6 tiles) against the CPU oracle: bit-exact int32 results, and
bit-exact dequantized outputs.

Every value of an INT4 operand is converted by a pre-pass into the workspace
and multiplied on v_mfma_scale_f32_32x32x64_f8f6f4, so each test compares the
whole output with the oracle.  Operands sit in buffers whose rows are wider
than K and padded with poison (0x77 bytes), and C sits in a sentinel-filled
guard buffer.  Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

POISON = gu.POISON["i4"]


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def device_operands(A, Bt, K, dev):
    lda_b = gu.round_up(K // 2, 16) + 16
    ldb_b = gu.round_up(K // 2, 16) + 32
    return (gu.to_device_padded(torch, A, lda_b, POISON, dev),
            gu.to_device_padded(torch, Bt, ldb_b, POISON, dev))


def run_f6(pd, dev, M, N, K, seed, cfg, rowb=False, scales=None, out_dtype=torch.int32):
    """One GEMM on an explicit FP6 tile (cfg) or, with cfg None, through the
    workspace entry point; returns host (A, B, C) with B as the operand passed
    (Bt column-major, or the row-major K x N packed along N)."""
    gu.note(f"[case] f6 M={M} N={N} K={K} seed={seed} cfg={cfg} rowb={rowb} "
            f"scales={scales is not None} out={out_dtype}")
    if rowb:
        A = synth.pack_int4(synth.int4_values(M, K, seed))
        Bv = synth.int4_values(N, K, seed + 1).T
        if N % 2:
            Bv = np.hstack([Bv, np.zeros((K, 1), np.int8)])
        B = synth.pack_int4(np.ascontiguousarray(Bv))
        Ad = gu.to_device_padded(torch, A, gu.round_up(K // 2, 16) + 16, POISON, dev)
        nb = B.shape[1]
        Bbuf = synth.with_leading_dim(np.vstack([B, np.full((2, nb), POISON, np.uint8)]),
                                      gu.round_up(nb, 16) + 16, POISON)
        Bd = torch.from_numpy(Bbuf).to(dev)[:K, :nb]
    else:
        A, B = synth.operands("i4", M, N, K, seed, seed + 1)
        Ad, Bd = device_operands(A, B, K, dev)
    ldc = gu.round_up(N, 4) + 4
    buf, out = gu.guarded_out(torch, M, N, ldc, out_dtype, dev)
    ws = pd.i4_workspace(M, N, K, dev, f6=True)
    if rowb:
        pd.gemm_i4_rowb(Ad, Bd, K, N, out=out, workspace=ws, f6cfg=cfg)
    elif scales is not None:
        sa, sb = (torch.from_numpy(x).to(dev) for x in scales)
        pd.gemm_i4_dequant(Ad, Bd, sa, sb, K, out=out, workspace=ws, f6cfg=cfg)
    elif cfg is None:
        pd.gemm_i4(Ad, Bd, K, out=out, workspace=ws)
    else:
        pd.gemm_i4(Ad, Bd, K, out=out, workspace=ws, f6cfg=cfg)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    return A, B, out.cpu().numpy()


def check(A, B, K, C, what, rowb=False):
    N = C.shape[1]
    if rowb:
        ref = oracle.gemm_i4_rowb(A, B, N=N, K=K)
    else:
        ref = oracle.gemm_i4(A, B, K=K)
    gu.assert_int_equal(C, ref, what)


# small, ragged and multi-tile shapes on every FP6 tile, compared in full
SHAPES = [(1, 1, 2), (2, 3, 8), (31, 33, 18), (33, 31, 130), (64, 64, 128), (65, 63, 256),
          (127, 129, 258), (255, 257, 384), (257, 255, 66), (300, 17, 1000), (17, 300, 1002),
          (520, 600, 520), (300, 260, 1030)]


@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_shapes_every_tile(pd, dev, cfg, shape):
    M, N, K = shape
    A, B, C = run_f6(pd, dev, M, N, K, 7000 + M + 3 * N + K, cfg)
    check(A, B, K, C, f"f6 cfg{cfg} {shape}")


ROWB_SHAPES = [(1, 1, 2), (31, 33, 18), (65, 63, 256), (127, 129, 258), (300, 17, 1000), (520, 601, 520)]


@pytest.mark.parametrize("cfg", [0, 1])
@pytest.mark.parametrize("shape", ROWB_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in ROWB_SHAPES])
def test_row_major_b(pd, dev, cfg, shape):
    M, N, K = shape
    A, B, C = run_f6(pd, dev, M, N, K, 8000 + M + N + K, cfg, rowb=True)
    check(A, B, K, C, f"f6 rowb cfg{cfg} {shape}", rowb=True)


@pytest.mark.parametrize("out", ["f32", "f16"])
@pytest.mark.parametrize("shape", [(33, 31, 130), (300, 260, 1030), (520, 600, 520)],
                         ids=["33x31x130", "300x260x1030", "520x600x520"])
def test_dequant(pd, dev, out, shape):
    M, N, K = shape
    sa, sb = synth.f32_scales(M, 91), synth.f32_scales(N, 92)
    dt = torch.float32 if out == "f32" else torch.float16
    A, B, C = run_f6(pd, dev, M, N, K, 9000 + M + N, 0, scales=(sa, sb), out_dtype=dt)
    want = oracle.dequant(oracle.gemm_i4(A, B, K=K), sa, sb, half_out=(out == "f16"))
    got = C.view(np.uint32 if out == "f32" else np.uint16)
    assert np.array_equal(got, want.view(got.dtype)), f"dequant {out} {shape}"


@pytest.mark.parametrize("cfg", [0, 1])
def test_largest_k_extremes(pd, dev, cfg):
    # K = 131070: every value -8 gives 64 K = 8388480, -8 against 7 gives -56 K;
    # the fp32 accumulators hold these integers exactly
    M, N, K = 130, 96, 131070
    gu.note(f"[case] f6 extremes K={K} cfg={cfg}")
    ws = pd.i4_workspace(M, N, K, dev, f6=True)
    ld = gu.round_up(K // 2, 16)   # rows span a multiple of 16 bytes
    p = lambda v, r: torch.from_numpy(
        synth.with_leading_dim(synth.pack_int4(np.full((r, K), v, np.int8)), ld, POISON)).to(dev)[:, :K // 2]
    for a, b, want in ((-8, -8, 64 * K), (-8, 7, -56 * K), (7, 7, 49 * K)):
        C = pd.gemm_i4(p(a, M), p(b, N), K, workspace=ws, f6cfg=cfg).cpu().numpy()
        assert np.all(C == want), (a, b)


@pytest.mark.parametrize("n", [2048, 4096, 8192])
def test_full_size_workspace_entry(pd, dev, n):
    """The sweep's INT4 GEMM (and config c2 at 4096) through the workspace entry
    point, in the launch the benchmark times: every element against the oracle,
    and bit equality with the INT8-MFMA kernel on the same operands."""
    cfg_id = 2 if n == 4096 else 4
    sa = synth.config_seed(cfg_id, n, synth.OPERAND_A)
    sb = synth.config_seed(cfg_id, n, synth.OPERAND_B)
    gu.note(f"[case] f6 full size {n}^3 seeds {sa:#x}/{sb:#x} pick={pd.i4_f6_pick(n, n, n)}")
    A, Bt = synth.operands("i4", n, n, n, sa, sb)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    ws = pd.i4_workspace(n, n, n, dev)
    C = torch.empty((n, n), dtype=torch.int32, device=dev)
    pd.prepare("i4", Ad, Bd, C, K=n, workspace=ws)
    Cp = pd.gemm_i4(Ad, Bd, n)
    torch.cuda.synchronize()
    assert torch.equal(C, Cp), "FP6 path differs from the INT8-MFMA path"
    C = C.cpu().numpy()
    del Ad, Bd, Cp, ws
    gu.check_whole("i4", A, Bt, n, C, f"f6 full {n}")


def test_workspace_errors(pd, dev):
    M = N = K = 4096
    gu.note("[case] f6 workspace errors")
    assert pd.i4_f6_pick(M, N, K) >= 0
    A = torch.zeros((M, K // 2), dtype=torch.uint8, device=dev)
    need = pd.i4_workspace_size(M, N, K)
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_i4(A, A, K, workspace=small)
    assert e.value.code == -7
    big = torch.empty(need + 32, dtype=torch.uint8, device=dev)
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_i4(A, A, K, workspace=big[8:8 + need])   # not 16-byte aligned
    assert e.value.code == -7
    # shapes of few tiles run the INT8-MFMA kernels and need no workspace
    assert pd.i4_workspace_size(64, 64, 4096) == 0
    Am = torch.zeros((64, K // 2), dtype=torch.uint8, device=dev)
    C = pd.gemm_i4(Am, Am, K, workspace=torch.empty(0, dtype=torch.uint8, device=dev))
    assert torch.count_nonzero(C) == 0


def test_repeat_and_reuse_workspace(pd, dev):
    # one workspace serves successive calls of different shapes, in order
    gu.note("[case] f6 workspace reuse")
    ws = pd.i4_workspace(1000, 700, 2050, dev, f6=True)
    for (M, N, K), seed in (((1000, 700, 2050), 1), ((300, 260, 1030), 2), ((1000, 700, 2050), 3)):
        A, Bt = synth.operands("i4", M, N, K, seed, seed + 1)
        Ad, Bd = device_operands(A, Bt, K, dev)
        C = pd.gemm_i4(Ad, Bd, K, workspace=ws, f6cfg=1).cpu().numpy()
        check(A, Bt, K, C, f"reuse {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# B converted once (i4_f6_pack), then GEMMs from A and B's image

def packed_case(pd, dev, M, N, K, seed, rowb=False, cfg=None, scales=None, out_dtype=torch.int32):
    gu.note(f"[case] packed B M={M} N={N} K={K} seed={seed} rowb={rowb} cfg={cfg} scales={scales is not None}")
    A = synth.pack_int4(synth.int4_values(M, K, seed))
    Ad = gu.to_device_padded(torch, A, gu.round_up(K // 2, 16) + 16, POISON, dev)
    if rowb:
        Bv = synth.int4_values(N, K, seed + 1).T
        if N % 2:
            Bv = np.hstack([Bv, np.zeros((K, 1), np.int8)])
        B = synth.pack_int4(np.ascontiguousarray(Bv))
        nb = B.shape[1]
        Bbuf = synth.with_leading_dim(np.vstack([B, np.full((2, nb), POISON, np.uint8)]),
                                      gu.round_up(nb, 16) + 16, POISON)
        img = pd.i4_f6_pack(torch.from_numpy(Bbuf).to(dev)[:K, :nb], K, rowmajor=True, N=N)
    else:
        B = synth.pack_int4(synth.int4_values(N, K, seed + 1))
        Bd = gu.to_device_padded(torch, B, gu.round_up(K // 2, 16) + 32, POISON, dev)
        img = pd.i4_f6_pack(Bd, K)
    buf, out = gu.guarded_out(torch, M, N, gu.round_up(N, 4) + 4, out_dtype, dev)
    sc = None if scales is None else tuple(torch.from_numpy(x).to(dev) for x in scales)
    pd.gemm_i4_packed_b(Ad, img, K, N, out=out, scales=sc, f6cfg=cfg)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    return A, B, out.cpu().numpy()


PACKED_SHAPES = [(1, 1, 2), (31, 33, 18), (65, 63, 256), (255, 257, 384), (300, 17, 1000), (520, 600, 520)]


@pytest.mark.parametrize("cfg", [None, 0, 1])
@pytest.mark.parametrize("rowb", [False, True], ids=["colB", "rowB"])
@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in PACKED_SHAPES])
def test_packed_b(pd, dev, cfg, rowb, shape):
    M, N, K = shape
    A, B, C = packed_case(pd, dev, M, N, K, 12000 + M + N + K, rowb=rowb, cfg=cfg)
    check(A, B, K, C, f"packed B {shape} rowb={rowb} cfg={cfg}", rowb=rowb)


@pytest.mark.parametrize("out", ["f32", "f16"])
def test_packed_b_dequant(pd, dev, out):
    M, N, K = 300, 260, 1030
    sa, sb = synth.f32_scales(M, 93), synth.f32_scales(N, 94)
    dt = torch.float32 if out == "f32" else torch.float16
    A, B, C = packed_case(pd, dev, M, N, K, 13000, scales=(sa, sb), out_dtype=dt)
    want = oracle.dequant(oracle.gemm_i4(A, B, K=K), sa, sb, half_out=(out == "f16"))
    got = C.view(np.uint32 if out == "f32" else np.uint16)
    assert np.array_equal(got, want.view(got.dtype)), f"packed dequant {out}"


def test_packed_b_image_serves_many_calls(pd, dev):
    """One image of an 8192 x 8192 B (as for a layer's weights) and GEMMs with
    A of 1024 and 2048 rows: bit-equal to gemm_i4 on the raw operands, and the
    first compared in full with the oracle."""
    N = K = 8192
    gu.note("[case] packed B 8192 x 8192 image, M = 1024 and 2048")
    Bt = synth.pack_int4(synth.int4_values(N, K, 14001))
    Bd = torch.from_numpy(Bt).to(dev)
    img = pd.i4_f6_pack(Bd, K)
    for M, seed in ((1024, 14002), (2048, 14003)):
        A = synth.pack_int4(synth.int4_values(M, K, seed))
        Ad = torch.from_numpy(A).to(dev)
        C = pd.gemm_i4_packed_b(Ad, img, K, N)
        ref = pd.gemm_i4(Ad, Bd, K)
        torch.cuda.synchronize()
        assert torch.equal(C, ref), f"packed B differs from gemm_i4 at M = {M}"
        if M == 1024:
            gu.check_whole("i4", A, Bt, K, C.cpu().numpy(), "packed B 1024 x 8192 x 8192")


def test_packed_b_errors(pd, dev):
    gu.note("[case] packed B errors")
    M, N, K = 64, 96, 256
    Bd = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev)
    img = pd.i4_f6_pack(Bd, K)
    Ad = torch.zeros((M, K // 2), dtype=torch.uint8, device=dev)
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_i4_packed_b(Ad, img[:img.numel() - 16], K, N)     # image for fewer rows or K
    assert e.value.code == -7
    with pytest.raises(pd.PdgemmError) as e:
        pd.i4_f6_pack(Bd, K, out=torch.empty(64, dtype=torch.uint8, device=dev))
    assert e.value.code == -7
