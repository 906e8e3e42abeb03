"""GPU parity of the dequantizing epilogue (INT8 / INT4 GEMM, then
C = ((float)S * scale_a[i]) * scale_b[j] in binary32, optionally rounded to
binary16) against the CPU oracle.

The result is unique (three binary32 roundings in a fixed order, then one
binary16 rounding), so every comparison is bit for bit: the output bits must
equal those the oracle computes from its own exact integer sums.  Scales are
seeded, positive and log-uniform (the per-row / per-column scales of a
symmetric quantization) unless a case says otherwise; operands are padded
with poison and outputs sit in a sentinel-filled buffer, as in the plain
GEMM's parity tests.  Every case prints its name before it touches the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

INT_PRECS = ("i8", "i4")
OUTS = ("f32", "f16")
SENTINEL16 = 0x7DAD  # a binary16 NaN pattern; never a result of finite scales


@pytest.fixture(scope="module")
def pd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_dense_gemm_amd as pd
    return pd


@pytest.fixture(scope="module")
def dev(pd):
    return torch.device("cuda:0")


def guarded(M, N, ldc, out, dev, extra_rows=3):
    """Sentinel-filled output buffer (M + extra_rows, ldc); returns (buf, view)."""
    if out == "f32":
        return gu.guarded_out(torch, M, N, ldc, torch.float32, dev, extra_rows)
    buf = torch.full((M + extra_rows, ldc), SENTINEL16, dtype=torch.int16, device=dev)
    buf = buf.view(torch.float16)
    return buf, buf[:M, :N]


def check_guard(buf, M, N, out):
    if out == "f32":
        return gu.check_guard(torch, buf, M, N)
    bits = buf.view(torch.int16).cpu().numpy()
    outside = np.ones(bits.shape, dtype=bool)
    outside[:M, :N] = False
    bad = np.count_nonzero(bits[outside] != np.int16(SENTINEL16))
    assert bad == 0, f"{bad} stores outside the M x N block"


def bits(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint16 if x.dtype == np.float16 else np.uint32)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.dtype == want.dtype, (got.dtype, want.dtype)
    g, w = bits(got), bits(want)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    same = (g == w) | nan_g  # NaN payloads are not part of the contract
    if not np.all(same):
        bad = np.argwhere(~same)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} "
                             f"({int(g[i]):#x}) want {want[i]!r} ({int(w[i]):#x})")


def oracle_dequant(prec, A, Bt, K, sa, sb, out):
    S = oracle.gemm_i8(A, Bt, K=K) if prec == "i8" else oracle.gemm_i4(A, Bt, K=K)
    return oracle.dequant(S, sa, sb, half_out=(out == "f16"))


def run_case(pd, dev, prec, M, N, K, seed, out, cfg=None, sa=None, sb=None, pad=True):
    """One dequantizing GEMM on padded, poisoned operands into a guarded output.
    Returns host (A, Bt, sa, sb, C)."""
    gu.note(f"[case] dequant {prec}->{out} M={M} N={N} K={K} seed={seed} cfg={cfg}")
    A, Bt = synth.operands(prec, M, N, K, seed, seed + 1)
    if sa is None:
        sa = synth.f32_scales(M, seed + 2)
    if sb is None:
        sb = synth.f32_scales(N, seed + 3)
    if prec == "i4":
        kb = K // 2
        Ad = gu.to_device_padded(torch, A, gu.round_up(kb, 16) + (16 if pad else 0), gu.POISON[prec], dev)
        Bd = gu.to_device_padded(torch, Bt, gu.round_up(kb, 16) + (32 if pad else 0), gu.POISON[prec], dev)
    else:
        Ad = gu.to_device_padded(torch, A, gu.round_up(K, 16) + (16 if pad else 0), gu.POISON[prec], dev)
        Bd = gu.to_device_padded(torch, Bt, gu.round_up(K, 16) + (32 if pad else 0), gu.POISON[prec], dev)
    # scale vectors sit one element into their buffers: only 4-byte alignment is promised
    sad = torch.from_numpy(np.concatenate([[np.float32(7)], sa]).astype(np.float32)).to(dev)[1:]
    sbd = torch.from_numpy(np.concatenate([[np.float32(7)], sb]).astype(np.float32)).to(dev)[1:]
    ldc = N + (3 if pad else 0)
    buf, outv = guarded(M, N, max(ldc, 1), out, dev, extra_rows=3 if pad else 0)
    if prec == "i8":
        pd.gemm_i8_dequant(Ad, Bd, sad, sbd, out=outv, cfg=cfg)
    else:
        pd.gemm_i4_dequant(Ad, Bd, sad, sbd, K, out=outv, cfg=cfg)
    torch.cuda.synchronize()
    check_guard(buf, M, N, out)
    return A, Bt, sa, sb, outv.cpu().numpy()


# ---------------------------------------------------------------------------
# small and ragged shapes, the library's own tile choice

SMALL = [(1, 1, 32), (2, 3, 64), (31, 33, 96), (65, 63, 130), (127, 129, 256),
         (255, 257, 258), (300, 17, 1000), (17, 300, 1002), (130, 70, 4096)]


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("prec", INT_PRECS)
@pytest.mark.parametrize("shape", SMALL, ids=[f"{m}x{n}x{k}" for m, n, k in SMALL])
def test_small_shapes(pd, dev, prec, out, shape):
    M, N, K = shape
    seed = 5000 + 7 * M + 13 * N + K
    A, Bt, sa, sb, C = run_case(pd, dev, prec, M, N, K, seed, out)
    assert_bits_equal(C, oracle_dequant(prec, A, Bt, K, sa, sb, out), f"{prec}->{out} {shape}")


# ---------------------------------------------------------------------------
# every tile configuration, several tiles and ragged tails

CFG_SHAPES = [(520, 600, 520), (300, 260, 1030)]


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("prec", INT_PRECS)
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
@pytest.mark.parametrize("shape", CFG_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in CFG_SHAPES])
def test_every_config(pd, dev, prec, out, cfg, shape):
    if cfg >= pd.num_configs():
        pytest.skip("configuration not present")
    M, N, K = shape
    A, Bt, sa, sb, C = run_case(pd, dev, prec, M, N, K, 91 + cfg, out, cfg=cfg)
    assert_bits_equal(C, oracle_dequant(prec, A, Bt, K, sa, sb, out), f"{prec}->{out} cfg{cfg} {shape}")


# ---------------------------------------------------------------------------
# closed forms and special values

@pytest.mark.parametrize("out", OUTS)
def test_closed_form_one(pd, dev, out):
    """All -128 (or all -8) operands: S = 16384 K (64 K); with scales 2^-14 (2^-6) and 1/K
    (a power of two) every output is exactly 1."""
    M, N, K = 130, 70, 1024
    gu.note(f"[case] dequant closed form ->{out}")
    odt = torch.float32 if out == "f32" else torch.float16
    i8 = lambda r: torch.full((r, K), -128, dtype=torch.int8, device=dev)
    sa = torch.full((M,), 2.0 ** -14, dtype=torch.float32, device=dev)
    sb = torch.full((N,), 1.0 / K, dtype=torch.float32, device=dev)
    C = pd.gemm_i8_dequant(i8(M), i8(N), sa, sb, out_dtype=odt).float().cpu().numpy()
    assert np.all(C == 1.0)
    p = lambda r: torch.from_numpy(synth.pack_int4(np.full((r, K), -8, np.int8))).to(dev)
    sa4 = torch.full((M,), 2.0 ** -6, dtype=torch.float32, device=dev)
    C = pd.gemm_i4_dequant(p(M), p(N), sa4, sb, K, out_dtype=odt).float().cpu().numpy()
    assert np.all(C == 1.0)


@pytest.mark.parametrize("prec", INT_PRECS)
@pytest.mark.parametrize("out", OUTS)
def test_signed_scales_and_special_values(pd, dev, prec, out):
    """Negative and zero scales (signed zeros), scales that overflow binary16 and
    binary32, subnormal results, and infinite scales (0 * inf = NaN)."""
    M, N, K = 96, 80, 200
    rng = np.random.default_rng(3)
    sa = (rng.uniform(-2, 2, M) * np.exp2(rng.integers(-60, 40, M))).astype(np.float32)
    sb = (rng.uniform(-2, 2, N) * np.exp2(rng.integers(-60, 40, N))).astype(np.float32)
    sa[:4] = [0.0, -0.0, np.inf, -np.inf]
    sb[:3] = [0.0, np.inf, 2.0 ** -149]
    A, Bt, sa, sb, C = run_case(pd, dev, prec, M, N, K, 17, out, sa=sa, sb=sb)
    want = oracle_dequant(prec, A, Bt, K, sa, sb, out)
    assert np.any(np.isinf(want)) and np.any(np.isnan(want)) and np.any(np.signbit(want) & (want == 0))
    assert_bits_equal(C, want, f"{prec}->{out} special values")


@pytest.mark.parametrize("prec", INT_PRECS)
def test_k_zero(pd, dev, prec):
    """K = 0: S = 0, so C = (0 * scale_a) * scale_b, signed zeros included."""
    M, N = 70, 90
    gu.note(f"[case] dequant {prec} K=0")
    dt = torch.int8 if prec == "i8" else torch.uint8
    A = torch.zeros((M, 16), dtype=dt, device=dev)[:, :0]
    B = torch.zeros((N, 16), dtype=dt, device=dev)[:, :0]
    sa = synth.f32_scales(M, 1) * np.where(np.arange(M) % 3 == 0, -1, 1).astype(np.float32)
    sb = synth.f32_scales(N, 2) * np.where(np.arange(N) % 5 == 0, -1, 1).astype(np.float32)
    sad, sbd = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    for out in OUTS:
        buf, outv = guarded(M, N, 96, out, dev)
        if prec == "i8":
            pd.gemm_i8_dequant(A, B, sad, sbd, out=outv)
        else:
            pd.gemm_i4_dequant(A, B, sad, sbd, 0, out=outv)
        torch.cuda.synchronize()
        check_guard(buf, M, N, out)
        want = oracle.dequant(np.zeros((M, N), np.int64), sa, sb, half_out=(out == "f16"))
        assert_bits_equal(outv.cpu().numpy(), want, f"{prec}->{out} K=0")


def test_f16_output_two_byte_aligned(pd, dev):
    """A binary16 output needs 2-byte alignment only: odd ldc and an odd element offset."""
    M, N, K = 50, 71, 96
    gu.note("[case] dequant f16 output, odd ldc and offset")
    A, Bt = synth.operands("i8", M, N, K, 3, 4)
    sa, sb = synth.f32_scales(M, 5), synth.f32_scales(N, 6)
    buf = torch.full((M, N + 1), SENTINEL16, dtype=torch.int16, device=dev).view(torch.float16)
    outv = buf[:, 1:]
    pd.gemm_i8_dequant(torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev),
                       torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev), out=outv)
    C = buf.cpu().numpy()
    assert np.all(C.view(np.int16)[:, 0] == np.int16(SENTINEL16))
    assert_bits_equal(C[:, 1:], oracle_dequant("i8", A, Bt, K, sa, sb, "f16"), "odd ldc")


# small M: the entry points pick the K-split tiles (3 = 32 x 32, 6 = 64 x 32)
KSPLIT = [((16, 520, 300), 3), ((1, 1000, 1030), 3), ((40, 8200, 260), 6), ((64, 8192, 130), 6)]


@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("prec", INT_PRECS)
@pytest.mark.parametrize("shape,cfg", KSPLIT, ids=[f"{m}x{n}x{k}" for (m, n, k), _ in KSPLIT])
def test_small_m_ksplit(pd, dev, prec, out, shape, cfg):
    M, N, K = shape
    assert pd.pick_config({"i8": 1, "i4": 2}[prec], M, N, K) == cfg
    A, Bt, sa, sb, C = run_case(pd, dev, prec, M, N, K, 12 + M, out)
    assert_bits_equal(C, oracle_dequant(prec, A, Bt, K, sa, sb, out), f"{prec}->{out} small M {shape}")


def test_scale_vector_errors(pd, dev):
    gu.note("[case] dequant binding errors")
    A = torch.zeros((8, 32), dtype=torch.int8, device=dev)
    s8 = torch.ones(8, device=dev)
    with pytest.raises(ValueError):
        pd.gemm_i8_dequant(A, A, s8, torch.ones(7, device=dev))
    with pytest.raises(TypeError):
        pd.gemm_i8_dequant(A, A, s8, torch.ones(8, dtype=torch.float64, device=dev))
    with pytest.raises(ValueError):
        pd.gemm_i8_dequant(A, A, s8, torch.ones(16, device=dev)[::2])
    with pytest.raises(TypeError):
        pd.gemm_i8_dequant(A, A, s8, s8, out=torch.empty((8, 8), dtype=torch.int32, device=dev))


# ---------------------------------------------------------------------------
# the raw sums are unchanged by the dequantizing path: unit scales give S
# rounded to binary32, i.e. exactly the plain GEMM's int32 result whenever
# |S| < 2^24

@pytest.mark.parametrize("prec", INT_PRECS)
def test_unit_scales_match_plain_gemm(pd, dev, prec):
    M, N, K = 300, 260, 512
    gu.note(f"[case] dequant {prec} unit scales vs plain")
    A, Bt = synth.operands(prec, M, N, K, 31, 32)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    one_a, one_b = torch.ones(M, device=dev), torch.ones(N, device=dev)
    if prec == "i8":
        S = pd.gemm_i8(Ad, Bd)
        C = pd.gemm_i8_dequant(Ad, Bd, one_a, one_b)
    else:
        S = pd.gemm_i4(Ad, Bd, K)
        C = pd.gemm_i4_dequant(Ad, Bd, one_a, one_b, K)
    S = S.cpu().numpy()
    assert np.abs(S).max() < 2 ** 24
    assert np.array_equal(C.cpu().numpy(), S.astype(np.float32))


# ---------------------------------------------------------------------------
# full size, in the launch the benchmark times (prepared, library tile choice):
# every element against the oracle, bit for bit

@pytest.mark.parametrize("prec", INT_PRECS)
@pytest.mark.parametrize("out", OUTS)
@pytest.mark.parametrize("M", [16, 64, 8192])
def test_full_size(pd, dev, prec, out, M):
    """M x 8192 x 8192 (the first M rows of the 8192^3 operands) in the launch the
    benchmark times; every element bit for bit."""
    n = 8192
    sa_seed = synth.config_seed(5, n, synth.OPERAND_A)
    sb_seed = synth.config_seed(5, n, synth.OPERAND_B)
    gu.note(f"[case] dequant {prec}->{out} {M}x{n}x{n} seeds {sa_seed:#x}/{sb_seed:#x}")
    A, Bt = synth.operands(prec, M, n, n, sa_seed, sb_seed)
    sa, sb = synth.f32_scales(M, sa_seed + 2), synth.f32_scales(n, sb_seed + 3)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
    sad, sbd = torch.from_numpy(sa).to(dev), torch.from_numpy(sb).to(dev)
    outv = torch.empty((M, n), dtype=torch.float32 if out == "f32" else torch.float16, device=dev)
    go = pd.prepare(prec, Ad, Bd, outv, K=n, scales=(sad, sbd))
    go()
    torch.cuda.synchronize()
    C = outv.cpu().numpy()
    del Ad, Bd, outv
    # every element: exact sums from the oracle's matrix-product form, then the
    # oracle's epilogue
    S = gu.oracle_whole(prec, A, Bt, n)
    want = oracle.dequant(S, sa, sb, half_out=(out == "f16"))
    assert_bits_equal(C, want, f"{prec}->{out} {M}x{n}x{n}")
    del S, want
    # and sampled entries with the sums from the triple loop
    rows, cols = gu.sample_positions(M, n, 512, seed=n + M)
    S = oracle.entries_i8(A, Bt, rows, cols) if prec == "i8" else oracle.entries_i4(A, Bt, rows, cols)
    want = oracle.dequant_entries(S, sa[rows], sb[cols], half_out=(out == "f16"))
    assert_bits_equal(C[rows, cols], want, f"{prec}->{out} {M}x{n}x{n} sampled")
