"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Integer results must be bit-exact; FP16 results must satisfy, per element,
|C - R| <= 1e-3 * S with R = sum_k a_ik b_kj and S = sum_k |a_ik b_kj| from
the oracle in fp64.  Every case prints its name, shape and seeds before it
touches the GPU.

Inputs come from ``synth`` with the distributions of the workloads: FP16
uniform on [-1, 1] (and N(0,1)/sqrt(K) for the 8192 case), INT8 uniform on
[-128, 127], INT4 uniform on [-8, 7].  Operands sit in buffers whose rows are
wider than K and padded with poison (NaN / 127 / 0x77), so a read past K
would show; outputs sit in a sentinel-filled buffer with extra rows and
columns, so a store outside M x N would show.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PRECS = ("f16", "i8", "i4")
NP_DTYPE = {"f16": np.float16, "i8": np.int8, "i4": np.uint8}


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def run_case(pd, dev, prec, M, N, K, seed, cfg=None, dist="uniform", pad=True, stream=None):
    """Run one GEMM on the GPU with padded/poisoned operands and a guarded output.
    Returns host (A, Bt, C) with A/Bt unpadded (packed for i4)."""
    gu.note(f"[case] {prec} M={M} N={N} K={K} seed={seed} cfg={cfg} dist={dist}")
    A, Bt = synth.operands(prec, M, N, K, seed, seed + 1, dist=dist)
    align = gu.ld_align(prec)
    if prec == "i4":
        kb = K // 2
        lda_b = gu.round_up(kb, 16) + (16 if pad else 0)
        ldb_b = gu.round_up(kb, 16) + (32 if pad else 0)
        Ad = gu.to_device_padded(torch, A, lda_b, gu.POISON[prec], dev)
        Bd = gu.to_device_padded(torch, Bt, ldb_b, gu.POISON[prec], dev)
    else:
        lda = gu.round_up(K, align) + (align if pad else 0)
        ldb = gu.round_up(K, align) + (2 * align if pad else 0)
        Ad = gu.to_device_padded(torch, A, max(lda, align), gu.POISON[prec], dev)
        Bd = gu.to_device_padded(torch, Bt, max(ldb, align), gu.POISON[prec], dev)
    ldc = gu.round_up(N, 4) + (4 if pad else 0)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    buf, out = gu.guarded_out(torch, M, N, max(ldc, 4), out_dtype, dev, extra_rows=3 if pad else 0)
    if prec == "f16":
        pd.gemm_f16(Ad, Bd, out=out, stream=stream, cfg=cfg)
    elif prec == "i8":
        pd.gemm_i8(Ad, Bd, out=out, stream=stream, cfg=cfg)
    else:
        pd.gemm_i4(Ad, Bd, K, out=out, stream=stream, cfg=cfg)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    C = out.cpu().numpy()
    return A, Bt, C


def check_full(prec, A, Bt, K, C, what):
    ref = gu.oracle_full(prec, A, Bt, K)
    if prec == "f16":
        gu.assert_f16_close(C, ref[0], ref[1], what)
    else:
        gu.assert_int_equal(C, ref, what)


# ---------------------------------------------------------------------------
# small and ragged shapes, full oracle comparison, default tile choice

SMALL_SHAPES = [
    (1, 1, 2), (1, 1, 64), (2, 3, 8), (16, 8, 16), (31, 33, 18), (33, 31, 34),
    (64, 64, 64), (65, 63, 130), (127, 129, 128), (128, 128, 256), (96, 80, 200),
    (255, 257, 258), (257, 255, 66), (300, 17, 1000), (17, 300, 1002),
]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SMALL_SHAPES])
def test_small_shapes(pd, dev, prec, shape):
    M, N, K = shape
    seed = 1000 + M * 7 + N * 13 + K
    A, Bt, C = run_case(pd, dev, prec, M, N, K, seed)
    check_full(prec, A, Bt, K, C, f"{prec} {shape}")


# ---------------------------------------------------------------------------
# every tile configuration, shapes spanning several tiles plus ragged tails

CFG_SHAPES = [(520, 600, 520), (300, 260, 1030), (64, 700, 130)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
@pytest.mark.parametrize("shape", CFG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in CFG_SHAPES])
def test_every_config(pd, dev, prec, cfg, shape):
    if cfg >= pd.num_configs():
        pytest.skip("configuration not present")
    M, N, K = shape
    A, Bt, C = run_case(pd, dev, prec, M, N, K, 77 + cfg, cfg=cfg)
    check_full(prec, A, Bt, K, C, f"{prec} cfg{cfg} {shape}")


# ---------------------------------------------------------------------------
# grids of whole 16 x 16 windows of tiles, where the tiles of band 4 (the
# 256-row tiles, and every tile of the 16 x 16 MFMA kernel) run in window
# order (one window per round, windows row by row in serpentine order): one
# window column, several in a row, 2 x 2 and 2 x 3 grids; every element checked

WINDOW_CASES = [(0, (4096, 8192, 320)), (0, (8192, 4096, 192)), (0, (8192, 12288, 96)),
                (4, (4096, 6144, 130)), (10, (4096, 8192, 200)), (1, (4096, 4096, 130)), (7, (2048, 6144, 64))]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("cfg,shape", WINDOW_CASES, ids=[f"cfg{c}-{m}x{n}x{k}" for c, (m, n, k) in WINDOW_CASES])
def test_window_order_grids(pd, dev, prec, cfg, shape):
    M, N, K = shape
    A, Bt, C = run_case(pd, dev, prec, M, N, K, 4242 + cfg, cfg=cfg)
    gu.check_whole(prec, A, Bt, K, C, f"{prec} cfg{cfg} {shape}")


# ---------------------------------------------------------------------------
# the worked example and closed forms on the GPU

def test_mma_lab_identity_on_gpu(pd, dev):
    """The 16x8x16 example of the PTX tutorial page ('Multiply one tile with a
    full warp'): A = I, B[r][c] = 8r + c + 1 gives C = B, and a row-reversing
    A puts 121..128 in the first row."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mma_lab_identity.json")))
    M, N, K = g["M"], g["N"], g["K"]
    B = np.array([[8 * r + c + 1 for c in range(N)] for r in range(K)], dtype=np.float16)
    Bt = torch.from_numpy(np.ascontiguousarray(B.T)).to(dev)
    A = torch.from_numpy(np.eye(M, K, dtype=np.float16)).to(dev)
    gu.note("[case] mma-lab identity 16x8x16")
    C = pd.gemm_f16(A, Bt).cpu().numpy()
    for r, c, v in g["printed_entries"]:
        assert C[r, c] == v
    assert np.array_equal(C, B.astype(np.float32))
    Ar = torch.from_numpy(np.ascontiguousarray(np.eye(M, K, dtype=np.float16)[::-1])).to(dev)
    C2 = pd.gemm_f16(Ar, Bt).cpu().numpy()
    assert list(C2[0]) == g["row_reversed_A_first_row"]


@pytest.mark.parametrize("K", [64, 2048, 8192])
def test_closed_form_extremes(pd, dev, K):
    M, N = 130, 70
    gu.note(f"[case] extremes K={K}")
    i8 = lambda v, r: torch.full((r, K), v, dtype=torch.int8, device=dev)
    C = pd.gemm_i8(i8(-128, M), i8(-128, N)).cpu().numpy()
    assert np.all(C == 16384 * K)
    C = pd.gemm_i8(i8(-128, M), i8(127, N)).cpu().numpy()
    assert np.all(C == -16256 * K)
    p = lambda v, r: torch.from_numpy(synth.pack_int4(np.full((r, K), v, np.int8))).to(dev)
    C = pd.gemm_i4(p(-8, M), p(-8, N), K).cpu().numpy()
    assert np.all(C == 64 * K)
    C = pd.gemm_i4(p(-8, M), p(7, N), K).cpu().numpy()
    assert np.all(C == -56 * K)
    C = pd.gemm_i4(p(7, M), p(7, N), K).cpu().numpy()
    assert np.all(C == 49 * K)
    ones = lambda r: torch.ones((r, K), dtype=torch.float16, device=dev)
    C = pd.gemm_f16(ones(M), ones(N)).cpu().numpy()
    assert np.all(C == K)


def test_identity_reproduces_operand(pd, dev):
    M, K = 200, 192
    gu.note("[case] right identity")
    A = synth.int8_matrix(M, K, 5)
    C = pd.gemm_i8(torch.from_numpy(A).to(dev), torch.eye(K, dtype=torch.int8, device=dev)).cpu().numpy()
    assert np.array_equal(C, A.astype(np.int32))
    A4 = synth.int4_values(M, K, 6)
    C = pd.gemm_i4(torch.from_numpy(synth.pack_int4(A4)).to(dev),
                   torch.from_numpy(synth.pack_int4(np.eye(K, dtype=np.int8))).to(dev), K).cpu().numpy()
    assert np.array_equal(C, A4.astype(np.int32))


# ---------------------------------------------------------------------------
# degenerate sizes and error paths

@pytest.mark.parametrize("prec", PRECS)
def test_k_zero_writes_zeros(pd, dev, prec):
    M, N = 70, 90
    gu.note(f"[case] {prec} K=0")
    buf, out = gu.guarded_out(torch, M, N, 96, torch.float32 if prec == "f16" else torch.int32, dev)
    dt = {"f16": torch.float16, "i8": torch.int8, "i4": torch.uint8}[prec]
    A = torch.zeros((M, 16), dtype=dt, device=dev)[:, :0]
    B = torch.zeros((N, 16), dtype=dt, device=dev)[:, :0]
    if prec == "f16":
        pd.gemm_f16(A, B, out=out)
    elif prec == "i8":
        pd.gemm_i8(A, B, out=out)
    else:
        pd.gemm_i4(A, B, 0, out=out)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    assert np.all(out.cpu().numpy() == 0)


def test_empty_outputs_are_noops(pd, dev):
    gu.note("[case] empty outputs")
    A = torch.zeros((0, 64), dtype=torch.int8, device=dev)
    B = torch.zeros((5, 64), dtype=torch.int8, device=dev)
    assert pd.gemm_i8(A, B).shape == (0, 5)
    assert pd.gemm_i8(B, A).shape == (5, 0)


def test_misaligned_operand_is_rejected(pd, dev):
    gu.note("[case] misaligned")
    buf = torch.zeros((64, 72), dtype=torch.float16, device=dev)
    B = torch.zeros((64, 64), dtype=torch.float16, device=dev)
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_f16(buf[:, 1:65], B)  # base pointer off by 2 bytes
    assert e.value.code == -5
    pd.gemm_f16(buf[:, :60], B[:, :60])  # lda 72 and ldb 64 are legal with K = 60
    Bw = torch.zeros((64, 68), dtype=torch.float16, device=dev)  # ldb 68: rows span 136 bytes
    with pytest.raises(pd.PdgemmError) as e:
        pd.gemm_f16(buf[:, :64], Bw[:, :64])
    assert e.value.code == -5


def test_unpadded_output_rows(pd, dev):
    # C needs no alignment beyond 4 bytes: ldc = N = 70 and an offset view work
    gu.note("[case] odd ldc")
    M, N, K = 50, 70, 96
    A, Bt = synth.operands("i8", M, N, K, 3, 4)
    buf = torch.full((M, N + 1), -7, dtype=torch.int32, device=dev)
    out = buf[:, 1:]
    pd.gemm_i8(torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev), out=out)
    C = buf.cpu().numpy()
    assert np.all(C[:, 0] == -7)
    gu.assert_int_equal(C[:, 1:], gu.oracle_full("i8", A, Bt, K), "odd ldc")


# ---------------------------------------------------------------------------
# determinism and streams

@pytest.mark.parametrize("prec", PRECS)
def test_repeatable_and_stream_independent(pd, dev, prec):
    M, N, K = 640, 384, 768
    gu.note(f"[case] {prec} determinism")
    A, Bt = synth.operands(prec, M, N, K, 9, 10)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    f = {"f16": pd.gemm_f16, "i8": pd.gemm_i8, "i4": lambda a, b, **kw: pd.gemm_i4(a, b, K, **kw)}[prec]
    ref = f(Ad, Bd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        others = [f(Ad, Bd) for _ in range(3)]
    torch.cuda.synchronize()
    for o in others:
        assert torch.equal(o.view(torch.int32), ref.view(torch.int32))


# ---------------------------------------------------------------------------
# the workloads at full size, in the launch configuration the benchmark uses
# (the entry points' own tile choice): every element against the oracle

FULL = [
    ("c0-f16-512", "f16", 512, "uniform", 0),
    ("c1-i8-2048", "i8", 2048, "uniform", 1),
    ("c2-i4-4096", "i4", 4096, "uniform", 2),
    ("c3-f16-8192-normal", "f16", 8192, "normal", 3),
] + [(f"c4-{p}-{n}", p, n, "uniform", 4) for p in PRECS for n in (512, 1024, 2048, 4096, 8192)]


@pytest.mark.parametrize("name,prec,n,dist,cfg_id", FULL, ids=[f[0] for f in FULL])
def test_workload_full_size(pd, dev, name, prec, n, dist, cfg_id):
    M = N = K = n
    sa = synth.config_seed(cfg_id, n, synth.OPERAND_A)
    sb = synth.config_seed(cfg_id, n, synth.OPERAND_B)
    gu.note(f"[case] {name}: {prec} {n}^3 seeds {sa:#x}/{sb:#x}")
    A, Bt = synth.operands(prec, M, N, K, sa, sb, dist=dist)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    if prec == "f16":
        C = pd.gemm_f16(Ad, Bd)
    elif prec == "i8":
        C = pd.gemm_i8(Ad, Bd)
    else:
        C = pd.gemm_i4(Ad, Bd, K)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    del Ad, Bd
    if n <= 1024:
        # the triple loop over the whole output
        check_full(prec, A, Bt, K, C, name)
    else:
        # every element against the oracle's matrix-product form, and sampled
        # entries plus tile edges against the triple loop as well
        gu.check_whole(prec, A, Bt, K, C, name)
        rows, cols = gu.sample_positions(M, N, 512, seed=n)
        gu.check_sampled(prec, A, Bt, K, C, rows, cols, name)


@pytest.mark.parametrize("prec", PRECS)
def test_prepared_launch_matches_plain_call(pd, dev, prec):
    M, N, K = 300, 260, 512
    gu.note(f"[case] {prec} prepared launch")
    A, Bt = synth.operands(prec, M, N, K, 21, 22)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    ref = torch.empty((M, N), dtype=out_dtype, device=dev)
    f = {"f16": pd.gemm_f16, "i8": pd.gemm_i8, "i4": lambda a, b, out: pd.gemm_i4(a, b, K, out=out)}[prec]
    f(Ad, Bd, out=ref)
    out = torch.full((M, N), -1, dtype=out_dtype, device=dev)
    go = pd.prepare(prec, Ad, Bd, out, K=K)
    for _ in range(3):
        go()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


# ---------------------------------------------------------------------------
# the K-split 32 x 32 tile (four waves per tile, each on its own quarter of
# every K tile, partials summed in wave order): small M or N

# (shape, the K-split tile the entry points pick: 3 = 32 x 32, 6 = 64 x 32)
KSPLIT_SHAPES = [((1, 1000, 3000), 3), ((16, 1000, 1030), 3), ((33, 700, 4100), 3), ((64, 257, 258), 3),
                 ((16, 96, 64), 3), ((5, 64, 2), 3), ((50, 8200, 700), 6), ((64, 8192, 1030), 6),
                 ((33, 8250, 130), 6)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("shape,cfg", KSPLIT_SHAPES, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in KSPLIT_SHAPES])
def test_ksplit_small_m(pd, dev, prec, shape, cfg):
    M, N, K = shape
    pnum = {"f16": 0, "i8": 1, "i4": 2}[prec]
    assert pd.pick_config(pnum, M, N, K) == cfg, "small M should take this K-split tile"
    A, Bt, C = run_case(pd, dev, prec, M, N, K, 4000 + M + N + K)
    check_full(prec, A, Bt, K, C, f"ksplit {prec} {shape}")


# one round of 64 x 64 tiles over a long K: configuration 9, four waves per
# tile on K slices (ragged in M, N and K), compared in full
LONG_K_SHAPES = [(128, 8192, 8192), (8192, 128, 8192), (120, 8190, 8448)]


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("shape", LONG_K_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in LONG_K_SHAPES])
def test_one_round_long_k(pd, dev, prec, shape):
    M, N, K = shape
    pnum = {"f16": 0, "i8": 1, "i4": 2}[prec]
    assert pd.pick_config(pnum, M, N, K) == 9, "one round of 64 x 64 tiles with K >= 8192 takes the K split"
    A, Bt, C = run_case(pd, dev, prec, M, N, K, 5000 + M + N + K)
    gu.check_whole(prec, A, Bt, K, C, f"long K {prec} {shape}")


def test_configs_without_k_split_give_the_same_fp16_bits(pd, dev):
    # every tile without a K split sums each element over K in the same order
    M, N, K = 300, 260, 1030
    gu.note("[case] f16 bits across configurations")
    A, Bt = synth.operands("f16", M, N, K, 61, 62)
    ld = gu.round_up(K, 8)
    Ad = torch.from_numpy(synth.with_leading_dim(A, ld)).to(dev)[:, :K]
    Bd = torch.from_numpy(synth.with_leading_dim(Bt, ld)).to(dev)[:, :K]
    info = {c: pd.config_info(c) for c in range(pd.num_configs())}
    plain = [c for c, v in info.items() if v["threads"] == (v["block_m"] // v["wave_m"]) * (v["block_n"] // v["wave_n"]) * 64]
    assert len(plain) >= 5
    outs = [pd.gemm_f16(Ad, Bd, cfg=c).view(torch.int32) for c in plain]
    for c, o in zip(plain[1:], outs[1:]):
        assert torch.equal(o, outs[0]), f"configuration {c} differs from {plain[0]}"


@pytest.mark.parametrize("cfg", [3, 6, 9])
def test_ksplit_f16_is_deterministic(pd, dev, cfg):
    # the partial tiles of the K split are summed in a fixed wave order
    M, N, K = 48, 2048, 4100
    gu.note(f"[case] ksplit f16 determinism cfg={cfg}")
    A, Bt = synth.operands("f16", M, N, K, 41, 42)
    ld = gu.round_up(K, 8)
    Ad = torch.from_numpy(synth.with_leading_dim(A, ld)).to(dev)[:, :K]
    Bd = torch.from_numpy(synth.with_leading_dim(Bt, ld)).to(dev)[:, :K]
    ref = pd.gemm_f16(Ad, Bd, cfg=cfg)
    for _ in range(3):
        assert torch.equal(pd.gemm_f16(Ad, Bd, cfg=cfg).view(torch.int32), ref.view(torch.int32))
    R, S = gu.oracle_full("f16", A, Bt, K)
    gu.assert_f16_close(ref.cpu().numpy(), R, S, f"ksplit determinism cfg{cfg}")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M", [16, 64])
def test_inference_shape_full_size(pd, dev, prec, M):
    """M x 8192 x 8192 in the launch the benchmark times: every element against the oracle."""
    n = 8192
    sa = synth.config_seed(7, n, synth.OPERAND_A)
    sb = synth.config_seed(7, n, synth.OPERAND_B)
    gu.note(f"[case] inference {prec} {M}x{n}x{n}")
    A, Bt = synth.operands(prec, M, n, n, sa, sb)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    C = torch.empty((M, n), dtype=torch.float32 if prec == "f16" else torch.int32, device=dev)
    pd.prepare(prec, Ad, Bd, C, K=n)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    gu.check_whole(prec, A, Bt, n, C, f"inference {prec} {M}")
    rows, cols = gu.sample_positions(M, n, 512, seed=M)
    gu.check_sampled(prec, A, Bt, n, C, rows, cols, f"inference {prec} {M}")
