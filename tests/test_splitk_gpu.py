"""GPU parity of the GEMM with K split across workgroups against the CPU oracle.

The split path zeroes the M x N block of C, then runs a grid with one row of
workgroups per range of K, each adding its partial tile into C with atomic
adds.  Integers must be bit-exact (integer addition is exact in any order);
FP16 takes two ranges and must stay within 1e-3 * sum |a*b| and give the
same bits on every call (binary32 addition commutes).  Operands sit in
poisoned padding and C in a sentinel-guarded buffer, so a read outside the
extents or a store outside the M x N block would show.  Every case prints its
name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import gpu_util as gu
from tests.test_rowb_gpu import oracle_rowb, rowb_operands

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PRECS = ("f16", "i8", "i4")
PREC_ID = {"f16": 0, "i8": 1, "i4": 2}


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def device_operands(prec, M, N, K, seed, rowb, dev):
    """Host operands (for the oracle) and their padded, poisoned device views."""
    poison = gu.POISON[prec]
    if rowb:
        A, B, _ = rowb_operands(prec, M, N, K, seed)
    else:
        A, B = synth.operands(prec, M, N, K, seed, seed + 1)
    if prec == "i4":
        ld_a = gu.round_up(K // 2, 16) + 16
        ld_b = gu.round_up(B.shape[1], 16) + 16
    else:
        al = gu.ld_align(prec)
        ld_a = gu.round_up(K, al) + al
        ld_b = gu.round_up(B.shape[1], al) + al
    Ad = gu.to_device_padded(torch, A, ld_a, poison, dev)
    Bbuf = np.full((B.shape[0] + 2, ld_b), poison, dtype=B.dtype)   # two poisoned rows past the end
    Bbuf[:B.shape[0], :B.shape[1]] = B
    if prec == "i4" and rowb and N % 2:
        # odd N: the high nibble of each row's last byte lies outside; poison it
        Bbuf[:K, B.shape[1] - 1] = (Bbuf[:K, B.shape[1] - 1] & 0x0F) | 0x70
    Bd = torch.from_numpy(Bbuf).to(dev)[:B.shape[0], :B.shape[1]]
    return A, B, Ad, Bd


def call(pd, prec, rowb, Ad, Bd, K, N, out, cfg=None, splits=None):
    if rowb:
        fn = {"f16": pd.gemm_f16_rowb, "i8": pd.gemm_i8_rowb}.get(prec)
        if fn is None:
            return pd.gemm_i4_rowb(Ad, Bd, K, N, out=out, cfg=cfg, splits=splits)
        return fn(Ad, Bd, out=out, cfg=cfg, splits=splits)
    if prec == "i4":
        return pd.gemm_i4(Ad, Bd, K, out=out, cfg=cfg, splits=splits)
    return (pd.gemm_f16 if prec == "f16" else pd.gemm_i8)(Ad, Bd, out=out, cfg=cfg, splits=splits)


def run(pd, dev, prec, M, N, K, seed, rowb, cfg=None, splits=None):
    gu.note(f"[case] splitk {prec} {'rowB' if rowb else 'colB'} M={M} N={N} K={K} seed={seed} "
            f"cfg={cfg} splits={splits}")
    A, B, Ad, Bd = device_operands(prec, M, N, K, seed, rowb, dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    buf, out = gu.guarded_out(torch, M, N, gu.round_up(N, 4) + 4, out_dtype, dev)
    call(pd, prec, rowb, Ad, Bd, K, N, out, cfg, splits)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    return A, B, out.cpu().numpy()


def reference(prec, A, B, K, N, rowb):
    if rowb:
        return oracle_rowb(prec, A, B, N, K)
    return gu.oracle_full(prec, A, B, K)


def check(prec, C, ref, what):
    if prec == "f16":
        gu.assert_f16_close(C, ref[0], ref[1], what)
    else:
        gu.assert_int_equal(C, ref, what)


# Ragged in every dimension.  K = 1030 / 2100 cut into ranges of whole
# 128-byte stages leave a last range that ends inside a stage (and, for
# i8 / i4 with 3 or 8 splits, inside a 16-byte chunk); splits = 8 on
# K = 1030 yields fewer ranges than asked.  K = 600 with the 64 x 64 tile and
# M = N = 1 is a single, partly masked tile per range.
SHAPES = [(70, 130, 1030), (130, 70, 2100), (1, 1, 600), (200, 333, 1030)]


@pytest.mark.parametrize("rowb", [False, True], ids=["colB", "rowB"])
@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("cfg", [2, 5])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in SHAPES])
def test_explicit_split(pd, dev, prec, rowb, cfg, shape):
    M, N, K = shape
    for splits in ([1, 2] if prec == "f16" else [2, 3, 8]):
        A, B, C = run(pd, dev, prec, M, N, K, 4100 + M + N + cfg, rowb, cfg=cfg, splits=splits)
        check(prec, C, reference(prec, A, B, K, N, rowb), f"splitk {prec} cfg{cfg} s{splits} {shape}")


@pytest.mark.parametrize("prec", PRECS)
def test_k_below_one_stage(pd, dev, prec):
    """K shorter than one stage: one range (the zero pass, then one atomic add per element)."""
    M, N, K = 65, 66, 32
    A, B, C = run(pd, dev, prec, M, N, K, 4200, True, cfg=2, splits=2)
    check(prec, C, reference(prec, A, B, K, N, True), f"splitk {prec} short K")


@pytest.mark.parametrize("prec", PRECS)
def test_k_zero(pd, dev, prec):
    M, N = 70, 96
    gu.note(f"[case] splitk {prec} K=0")
    dt = {"f16": torch.float16, "i8": torch.int8, "i4": torch.uint8}[prec]
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    buf, out = gu.guarded_out(torch, M, N, 100, out_dtype, dev)
    A = torch.zeros((M, 16), dtype=dt, device=dev)[:, :0]
    Bt = torch.zeros((N, 16), dtype=dt, device=dev)[:, :0]
    call(pd, prec, False, A, Bt, 0, N, out, cfg=2, splits=2)
    torch.cuda.synchronize()
    gu.check_guard(torch, buf, M, N)
    assert np.all(out.cpu().numpy() == 0)


# Shapes the entry points split (few 64 x 64 tiles, long K), each with the
# (ranges, tile) pick_splits must give: row-major B at M <= 64 over wide and
# narrow N, 128 x 64 tiles past 64 rows, column-major B with at most 32 tiles.
AUTO = [("i8", True, (64, 8192, 8192), (2, 2)), ("i4", True, (16, 8192, 8192), (2, 2)),
        ("i8", True, (16, 2048, 16384), (8, 2)), ("i4", True, (64, 4096, 16384), (4, 2)),
        ("i8", True, (512, 1024, 32768), (4, 5)), ("i4", True, (96, 4096, 16384), (4, 5)),
        ("i8", False, (64, 2048, 32768), (8, 2)), ("i4", False, (512, 512, 65536), (8, 5)),
        ("f16", True, (16, 4096, 16384), (2, 2)), ("f16", True, (100, 2048, 16384), (2, 2))]


@pytest.mark.parametrize("prec,rowb,shape,plan", AUTO,
                         ids=[f"{p}-{'rowB' if r else 'colB'}-{m}x{n}x{k}" for p, r, (m, n, k), _ in AUTO])
def test_entry_point_split_full_size(pd, dev, prec, rowb, shape, plan):
    """The picked split at full size: every element against the oracle's matrix-product form."""
    M, N, K = shape
    assert pd.pick_splits(PREC_ID[prec], M, N, K, rowb=rowb) == plan
    A, B, C = run(pd, dev, prec, M, N, K, 4500 + M + N, rowb)
    gu.check_whole(prec, A, B, K, C, f"splitk entry {prec} {shape}", rowb=rowb)


def test_f16_split_same_bits_every_call(pd, dev):
    """Two ranges added atomically: the same bits whichever range lands first."""
    M, N, K = 16, 4096, 16384
    gu.note(f"[case] splitk f16 determinism {M}x{N}x{K}")
    A, B, Ad, Bd = device_operands("f16", M, N, K, 4300, True, dev)
    assert pd.pick_splits(0, M, N, K, rowb=True) == (2, 2)
    first = pd.gemm_f16_rowb(Ad, Bd).cpu().numpy()
    for _ in range(4):
        again = pd.gemm_f16_rowb(Ad, Bd).cpu().numpy()
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_i4_longest_k_closed_form(pd, dev):
    """INT4 at its largest K, split eight ways: (-8) * 7 summed 131070 times."""
    M, N, K = 16, 256, 131070
    gu.note(f"[case] splitk i4 longest K {M}x{N}x{K}")
    assert pd.pick_splits(2, M, N, K, rowb=True) == (8, 2)
    # rows of A span K / 2 = 65535 bytes: a view of a buffer 65536 bytes wide
    a = torch.from_numpy(synth.pack_int4(np.full((M, K + 2), -8, np.int8))).to(dev)[:, :K // 2]
    b = torch.from_numpy(synth.pack_int4(np.full((K, N), 7, np.int8))).to(dev)
    assert np.all(pd.gemm_i4_rowb(a, b, K, N).cpu().numpy() == -56 * K)


@pytest.mark.parametrize("prec", PRECS)
def test_graph_replays(pd, dev, prec):
    """The zero pass and the atomic GEMM captured in a graph: each replay, after
    eager work that overwrites C, gives the eager result again."""
    M, N, K = 32, 2048, 16384
    rowb = True
    plan = pd.pick_splits(PREC_ID[prec], M, N, K, rowb=rowb)
    assert plan[0] > 1
    gu.note(f"[case] splitk graph {prec} {M}x{N}x{K} plan {plan}")
    A, B, Ad, Bd = device_operands(prec, M, N, K, 4400, rowb, dev)
    out_dtype = torch.float32 if prec == "f16" else torch.int32
    out = torch.empty((M, N), dtype=out_dtype, device=dev)
    eager = call(pd, prec, rowb, Ad, Bd, K, N, out).cpu().numpy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(pd, prec, rowb, Ad, Bd, K, N, out)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep} differs"
    gu.check_whole(prec, A, B, K, eager, f"splitk graph {prec}", rowb=rowb)
