"""C-ABI checks that need no GPU: the library loads, exports every function
that include/pdgemm.h declares, and rejects bad arguments on the host before
any HIP call (dummy, never-dereferenced pointers are enough for that)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pdgemm.h")
LIB = os.path.join(ROOT, "precision_dense_gemm_amd", "libpdgemm.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpdgemm.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def codes():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(PDGEMM_E\w+|PDGEMM_OK)\s+\(?(-?\d+)\)?", text)}


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    for name in ("gemm_f16", "gemm_i8", "gemm_i4"):
        getattr(L, name).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
        getattr(L, name).restype = i
    for name in ("gemm_i8_dequant", "gemm_i4_dequant"):
        getattr(L, name).argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p]
        getattr(L, name).restype = i
    for name in ("gemm_f16_rowb", "gemm_i8_rowb", "gemm_i4_rowb"):
        getattr(L, name).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
        getattr(L, name).restype = i
    L.pdgemm_gemm_rowb_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.pdgemm_gemm_rowb_cfg.restype = i
    L.pdgemm_dequant_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p]
    L.pdgemm_dequant_cfg.restype = i
    L.pdgemm_gemm_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.pdgemm_gemm_cfg.restype = i
    L.pdgemm_strerror.argtypes = [i]
    L.pdgemm_strerror.restype = ctypes.c_char_p
    L.pdgemm_pick_config.argtypes = [i, i64, i64, i64]
    L.pdgemm_config_info.argtypes = [i] + [ctypes.POINTER(i)] * 5
    return L


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gemm_f16", "gemm_i8", "gemm_i4", "gemm_i8_dequant", "gemm_i4_dequant",
              "gemm_f16_rowb", "gemm_i8_rowb", "gemm_i4_rowb", "pdgemm_gemm_rowb_cfg",
              "pdgemm_gemm_cfg", "pdgemm_dequant_cfg", "pdgemm_strerror", "pdgemm_version",
              "gemm_i4_ws", "gemm_i4_rowb_ws", "gemm_i4_dequant_ws", "pdgemm_i4_workspace_size",
              "pdgemm_i4_f6_cfg", "pdgemm_i4_f6_pick", "pdgemm_i4_f6_num_configs",
              "pdgemm_i4_f6_workspace_bytes", "pdgemm_i4_f6_image_bytes", "pdgemm_i4_f6_pack",
              "gemm_i4_packed_b", "gemm_i4_dequant_packed_b", "pdgemm_i4_packed_b_cfg",
              "gemm_i4_noalloc", "pdgemm_i4_noalloc_max_bytes"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        getattr(lib, name)  # resolvable through the dynamic loader


def test_no_torch_or_oracle_in_the_library():
    out = subprocess.run(["ldd", LIB], capture_output=True, text=True).stdout
    assert "torch" not in out and "oracle" not in out
    out = subprocess.run(["nm", "-D", LIB], capture_output=True, text=True).stdout
    assert "oracle_" not in out


# dummy device pointers: 16-byte aligned, never dereferenced by the host checks
PA, PB, PC = 0x10000, 0x20000, 0x30000


def call(lib, name, M, N, K, A=PA, lda=None, B=PB, ldb=None, C=PC, ldc=None):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return getattr(lib, name)(M, N, K, A, lda, B, ldb, C, ldc, None)


@pytest.mark.parametrize("name", ["gemm_f16", "gemm_i8", "gemm_i4"])
def test_argument_errors(lib, name):
    c = codes()
    assert call(lib, name, -1, 64, 64) == c["PDGEMM_EINVAL_DIM"]
    assert call(lib, name, 64, -1, 64) == c["PDGEMM_EINVAL_DIM"]
    assert call(lib, name, 64, 64, -2) == c["PDGEMM_EINVAL_DIM"]
    assert call(lib, name, 64, 64, 64, lda=32) == c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, 64, 64, 64, ldb=32) == c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, 64, 64, 64, ldc=32) == c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, 64, 64, 64, A=None) == c["PDGEMM_ENULL"]
    assert call(lib, name, 64, 64, 64, B=None) == c["PDGEMM_ENULL"]
    assert call(lib, name, 64, 64, 64, C=None) == c["PDGEMM_ENULL"]
    # misaligned base pointers and leading dimensions
    assert call(lib, name, 64, 64, 64, A=PA + 2) == c["PDGEMM_EALIGN"]
    assert call(lib, name, 64, 64, 64, B=PB + 8) == c["PDGEMM_EALIGN"]
    assert call(lib, name, 64, 64, 64, C=PC + 2) == c["PDGEMM_EALIGN"]
    # empty outputs are a no-op that succeeds without touching HIP
    assert call(lib, name, 0, 64, 64) == 0
    assert call(lib, name, 64, 0, 64) == 0
    assert call(lib, name, 0, 0, 0, A=None, B=None, C=None) == 0


PSA, PSB = 0x40000, 0x50000


def call_dq(lib, name, M, N, K, A=PA, lda=None, B=PB, ldb=None, sa=PSA, sb=PSB, C=PC, ldc=None,
            f16=0):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return getattr(lib, name)(M, N, K, A, lda, B, ldb, sa, sb, C, ldc, f16, None)


@pytest.mark.parametrize("name", ["gemm_i8_dequant", "gemm_i4_dequant"])
def test_dequant_argument_errors(lib, name):
    c = codes()
    assert call_dq(lib, name, -1, 64, 64) == c["PDGEMM_EINVAL_DIM"]
    assert call_dq(lib, name, 64, 64, 64, lda=32) == c["PDGEMM_EINVAL_LD"]
    assert call_dq(lib, name, 64, 64, 64, ldc=32) == c["PDGEMM_EINVAL_LD"]
    assert call_dq(lib, name, 64, 64, 64, A=None) == c["PDGEMM_ENULL"]
    assert call_dq(lib, name, 64, 64, 64, C=None) == c["PDGEMM_ENULL"]
    assert call_dq(lib, name, 64, 64, 64, sa=None) == c["PDGEMM_ENULL"]
    assert call_dq(lib, name, 64, 64, 64, sb=None) == c["PDGEMM_ENULL"]
    assert call_dq(lib, name, 64, 64, 0, A=None, B=None, sa=None) == c["PDGEMM_ENULL"]
    # scales are element-aligned; a binary16 output needs only 2 bytes
    assert call_dq(lib, name, 64, 64, 64, sa=PSA + 2) == c["PDGEMM_EALIGN"]
    assert call_dq(lib, name, 64, 64, 64, sb=PSB + 1) == c["PDGEMM_EALIGN"]
    assert call_dq(lib, name, 64, 64, 64, C=PC + 2) == c["PDGEMM_EALIGN"]
    assert call_dq(lib, name, 64, 64, 64, C=PC + 1, f16=1) == c["PDGEMM_EALIGN"]
    # a row of C above 4 MiB: the byte span depends on the output type
    assert call_dq(lib, name, 64, 64, 64, ldc=(1 << 20) + 64) == c["PDGEMM_EINVAL_LD"]
    assert call_dq(lib, name, 64, 64, 64, ldc=(1 << 21) + 64, f16=1) == c["PDGEMM_EINVAL_LD"]
    # empty outputs succeed without touching HIP, scales unused
    assert call_dq(lib, name, 0, 64, 64, sa=None, sb=None) == 0
    assert call_dq(lib, name, 64, 0, 64, sa=None, sb=None) == 0
    if name == "gemm_i4_dequant":
        assert call_dq(lib, name, 64, 64, 63, lda=64, ldb=64) == c["PDGEMM_EINVAL_I4"]


@pytest.mark.parametrize("name", ["gemm_f16_rowb", "gemm_i8_rowb", "gemm_i4_rowb"])
def test_rowb_argument_errors(lib, name):
    c = codes()
    # a row of row-major B holds N values: ldb >= N, independent of K
    assert call(lib, name, 64, 96, 64, ldb=64) == c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, 64, 64, 96, ldb=64) != c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, 64, 64, 64, lda=32) == c["PDGEMM_EINVAL_LD"]
    assert call(lib, name, -1, 64, 64) == c["PDGEMM_EINVAL_DIM"]
    assert call(lib, name, 64, 64, 64, B=None) == c["PDGEMM_ENULL"]
    assert call(lib, name, 64, 64, 64, B=PB + 8) == c["PDGEMM_EALIGN"]
    assert call(lib, name, 64, 60, 64, ldb=60) == c["PDGEMM_EALIGN"]  # rows of B span 16-byte multiples
    assert call(lib, name, 0, 64, 64) == 0
    if name == "gemm_i4_rowb":
        assert call(lib, name, 64, 64, 64, ldb=65) == c["PDGEMM_EINVAL_I4"]
        assert call(lib, name, 64, 64, 63, lda=64, ldb=64) == c["PDGEMM_EINVAL_I4"]
    n = lib.pdgemm_num_configs()
    assert lib.pdgemm_gemm_rowb_cfg(0, n, 64, 64, 64, PA, 64, PB, 64, PC, 64, None) == c["PDGEMM_EINVAL_CFG"]


def test_dequant_cfg_errors(lib):
    c = codes()
    n = lib.pdgemm_num_configs()
    args = (64, 64, 64, PA, 64, PB, 64, PSA, PSB, PC, 64, 0, None)
    assert lib.pdgemm_dequant_cfg(0, 0, *args) == c["PDGEMM_EINVAL_CFG"]   # FP16 has no dequant
    assert lib.pdgemm_dequant_cfg(1, n, *args) == c["PDGEMM_EINVAL_CFG"]
    assert lib.pdgemm_dequant_cfg(2, -1, *args) == c["PDGEMM_EINVAL_CFG"]
    assert lib.pdgemm_dequant_cfg(3, 0, *args) == c["PDGEMM_EINVAL_CFG"]
    # every variant exists on the K-split tiles; argument errors are found before any HIP call
    ks = [cfg for cfg in range(n) if _k_split(lib, cfg) > 1]
    assert ks, "no K-split configuration"
    for cfg in ks:
        assert lib.pdgemm_gemm_rowb_cfg(1, cfg, 64, 64, 64, PA, 64, None, 64, PC, 64, None) == c["PDGEMM_ENULL"]
        assert lib.pdgemm_dequant_cfg(1, cfg, 64, 64, 64, PA, 64, PB, 64, None, PSB, PC, 64, 0,
                                      None) == c["PDGEMM_ENULL"]


def _k_split(lib, cfg):
    """Waves per output wave tile: threads / (waves tiling the block * 64)."""
    vals = [ctypes.c_int() for _ in range(5)]
    assert lib.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals]) == 0
    bm, bn, wm, wn, threads = (v.value for v in vals)
    return threads // ((bm // wm) * (bn // wn) * 64)


def test_grid_beyond_32_bit_work_items_is_rejected(lib):
    c = codes()
    # 2^20 x 2^20 outputs on 64 x 64 tiles: 2^28 workgroups of 256 work-items
    big = 1 << 20
    assert lib.pdgemm_gemm_cfg(1, 2, big, big, 64, PA, 64, PB, 64, PC, big, None) == c["PDGEMM_EINVAL_DIM"]
    assert lib.pdgemm_gemm_cfg(1, 2, 64, 64, 1 << 31, PA, 1 << 31, PB, 1 << 31, PC, 64, None) == c["PDGEMM_EINVAL_DIM"]


def test_alignment_of_leading_dims_per_precision(lib):
    c = codes()
    # f16 rows must span multiples of 8 elements, i8 of 16, i4 of 32
    assert call(lib, "gemm_f16", 64, 64, 60, lda=60) == c["PDGEMM_EALIGN"]
    assert call(lib, "gemm_i8", 64, 64, 60, lda=60) == c["PDGEMM_EALIGN"]
    assert call(lib, "gemm_i4", 64, 64, 60, lda=60) == c["PDGEMM_EALIGN"]
    assert call(lib, "gemm_i4", 64, 64, 48, lda=48) == c["PDGEMM_EALIGN"]


def test_int4_specific_errors(lib):
    c = codes()
    assert call(lib, "gemm_i4", 64, 64, 63, lda=64, ldb=64) == c["PDGEMM_EINVAL_I4"]
    assert call(lib, "gemm_i4", 64, 64, 64, lda=65) == c["PDGEMM_EINVAL_I4"]
    assert call(lib, "gemm_i4", 64, 64, 131072) == c["PDGEMM_EINVAL_DIM"]


def test_config_errors_and_info(lib):
    c = codes()
    n = lib.pdgemm_num_configs()
    assert n >= 1
    assert lib.pdgemm_gemm_cfg(0, n, 64, 64, 64, PA, 64, PB, 64, PC, 64, None) == c["PDGEMM_EINVAL_CFG"]
    assert lib.pdgemm_gemm_cfg(3, 0, 64, 64, 64, PA, 64, PB, 64, PC, 64, None) == c["PDGEMM_EINVAL_CFG"]
    assert lib.pdgemm_gemm_cfg(0, -1, 64, 64, 64, PA, 64, PB, 64, PC, 64, None) == c["PDGEMM_EINVAL_CFG"]
    for cfg in range(n):
        vals = [ctypes.c_int() for _ in range(5)]
        assert lib.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals]) == 0
        bm, bn, wm, wn, threads = (v.value for v in vals)
        assert bm % wm == 0 and bn % wn == 0 and wm % 32 == 0 and wn % 32 == 0
        # waves tile the block, times the K split (4 waves share one 32 x 32 tile)
        assert threads in ((bm // wm) * (bn // wn) * 64, (bm // wm) * (bn // wn) * 64 * 4)
    assert lib.pdgemm_config_info(n, None, None, None, None, None) == c["PDGEMM_EINVAL_CFG"]
    for prec in (0, 1, 2):
        for size in (1, 512, 2048, 8192):
            assert 0 <= lib.pdgemm_pick_config(prec, size, size, size) < n
    assert lib.pdgemm_pick_config(7, 64, 64, 64) == -1


def test_strerror_and_version(lib):
    for name, code in codes().items():
        msg = lib.pdgemm_strerror(code)
        assert msg and len(msg) > 3, name
    assert lib.pdgemm_strerror(-999)
    assert lib.pdgemm_version() >= 200


def test_binding_imports_and_marshals_without_gpu():
    import torch
    import precision_dense_gemm_amd as pd
    assert pd.version() == pd.lib.pdgemm_version()
    assert pd.config_info(0)["threads"] > 0
    with pytest.raises(TypeError):
        pd.gemm_i8(torch.zeros(4, 4, dtype=torch.float16), torch.zeros(4, 4, dtype=torch.int8))
    with pytest.raises(ValueError):
        pd.gemm_i8(torch.zeros(4, 4, dtype=torch.int8), torch.zeros(4, 4, dtype=torch.int8))  # CPU tensors
    with pytest.raises(TypeError):
        pd.gemm_i8_dequant(torch.zeros(4, 4, dtype=torch.float16), torch.zeros(4, 4, dtype=torch.int8),
                           torch.ones(4), torch.ones(4))


def test_pick_prefers_large_tiles_that_fill_the_chip(lib):
    # square sizes of the sweep keep their tiles; a wide product with few rows takes
    # the intermediate tiles, and small M the K-split tile
    info = {}
    for cfg in range(lib.pdgemm_num_configs()):
        vals = [ctypes.c_int() for _ in range(5)]
        assert lib.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals]) == 0
        info[cfg] = tuple(v.value for v in vals)
    def tile(m, n, k=8192):
        c = lib.pdgemm_pick_config(1, m, n, k)
        return info[c][:2], c
    assert tile(8192, 8192)[0] == (256, 256)
    assert tile(4096, 4096)[0] == (256, 256)
    assert tile(2048, 2048)[0] == (128, 128)
    assert tile(1024, 1024)[0] == (64, 64)
    assert tile(1024, 8192)[0] == (256, 128)
    # 256 x 8192 x 8192: a full round of 128 x 64 rather than 128 tiles of 128 x 128, which
    # would busy exactly half of the CUs (timed slower, most with row-major B)
    assert tile(256, 8192)[0] == (128, 64)
    assert tile(16, 8192)[0] == (32, 32) and _k_split(lib, tile(16, 8192)[1]) == 4
    assert tile(64, 8192)[0] == (64, 32) and _k_split(lib, tile(64, 8192)[1]) == 4
    assert tile(512, 512)[0] == (32, 32)
    for m, n in ((1024, 8192), (256, 8192), (16, 8192), (8192, 8192), (512, 512)):
        bm, bn = tile(m, n)[0]
        assert -(-m // bm) * -(-n // bn) >= 256
    # INT4 too takes 256 x 128 here (with 8 waves it overlaps its unpack with the MFMAs)
    assert info[lib.pdgemm_pick_config(2, 1024, 8192, 8192)][:2] == (256, 128)


def test_pick_weighs_the_last_partial_round(lib):
    # Measured optima (medians of alternated timings of every tile) where the
    # largest tile that fills the chip is not the fastest: fewer, larger tiles
    # when the larger one still busies most CUs, and a smaller tile when the
    # larger one would leave a last round mostly empty.
    info = {}
    for cfg in range(lib.pdgemm_num_configs()):
        vals = [ctypes.c_int() for _ in range(5)]
        lib.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals])
        info[cfg] = tuple(v.value for v in vals)[:2]
    def tile(prec, m, n, k):
        return info[lib.pdgemm_pick_config(prec, m, n, k)]
    for prec in range(3):
        assert tile(prec, 3584, 3584, 3584) == (256, 256)     # 196 tiles, not 392 of 256 x 128
        assert tile(prec, 3072, 3072, 3072) == (256, 256)     # 144 tiles, not 2.25 rounds of 128 x 128
        assert tile(prec, 1792, 8192, 8192) == (256, 256)     # 224 tiles
        assert tile(prec, 8192, 8192, 8192) == (256, 256)
        assert tile(prec, 12288, 4096, 4096) == (256, 256)
        assert tile(prec, 5120, 5120, 5120) == (256, 256)     # 400 tiles: 1.56 rounds
        assert tile(prec, 7168, 7168, 7168) == (256, 256)
        assert tile(prec, 1024, 8192, 8192) == (256, 128)     # 128 tiles of 256 x 256 would idle half the CUs
        assert tile(prec, 1536, 4096, 8192) == (256, 128)
    for prec in (0, 1):
        assert tile(prec, 6144, 6144, 6144) == (256, 256)     # 2.25 rounds beat 4.5 of 256 x 128
    # one round of 64 x 64 tiles over a long K splits K over the four waves of each tile
    for prec in range(3):
        assert lib.pdgemm_pick_config(prec, 128, 8192, 8192) == 9
        assert lib.pdgemm_pick_config(prec, 8192, 128, 8192) == 9
        assert tile(prec, 128, 8192, 4096) == (64, 64) and lib.pdgemm_pick_config(prec, 128, 8192, 4096) == 2
        assert lib.pdgemm_pick_config(prec, 1024, 1024, 1024) == 2
        assert lib.pdgemm_pick_config(prec, 128, 8192, 8224) == 2   # rows of K end inside a 128-byte line
    # 128 x 128 at one tile per CU takes its three-stage variant; with more tiles, two stages
    three_stage = lib.pdgemm_pick_config(0, 2048, 2048, 2048)
    assert info[three_stage] == (128, 128)
    assert info[lib.pdgemm_pick_config(2, 10240, 2048, 4096)] == (128, 128)   # INT4: 1280 tiles
    assert lib.pdgemm_pick_config(2, 10240, 2048, 4096) != three_stage
    # whenever the 64 x 64 tile fills the chip, the pick gives at least half of the CUs a tile
    for prec in range(3):
        for m in range(512, 12289, 448):
            for n in range(512, 12289, 704):
                bm, bn = tile(prec, m, n, 4096)
                if -(-m // 64) * -(-n // 64) >= 256:
                    assert -(-m // bm) * -(-n // bn) >= 128, (prec, m, n)


@pytest.fixture(scope="module")
def sklib(lib):
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.pdgemm_pick_splits.argtypes = [i, i, i64, i64, i64, ctypes.POINTER(i)]
    lib.pdgemm_pick_splits.restype = i
    lib.pdgemm_gemm_splitk_cfg.argtypes = [i, i, i, i, i64, i64, i64, p, i64, p, i64, p, i64, p]
    lib.pdgemm_gemm_splitk_cfg.restype = i
    return lib


def splits_of(lib, prec, rowb, m, n, k):
    cfg = ctypes.c_int()
    s = lib.pdgemm_pick_splits(prec, rowb, m, n, k, ctypes.byref(cfg))
    return s, cfg.value


def test_pick_splits_where_measured(sklib):
    L = sklib
    # measured gains (row-major B unless noted): 1.2-1.3x, 1.7x, 3x, 1.7x, 1.7x (column-major), 1.2x (FP16)
    assert splits_of(L, 1, 1, 64, 8192, 8192) == (2, 2)
    assert splits_of(L, 2, 1, 16, 8192, 8192) == (2, 2)
    assert splits_of(L, 2, 1, 16, 4096, 16384) == (4, 2)
    assert splits_of(L, 1, 1, 64, 2048, 32768) == (8, 2)
    assert splits_of(L, 1, 1, 512, 1024, 32768) == (4, 5)    # 128 x 64 tiles past 64 rows of A
    assert splits_of(L, 1, 0, 64, 2048, 32768) == (8, 2)
    assert splits_of(L, 0, 1, 16, 4096, 16384) == (2, 2)
    # measured losses the rule declines: short K, a chip already filled, the
    # one-round K-split tile, column-major B over more than 32 tiles, FP16
    # below K = 16384 or with column-major B
    for prec, rowb, m, n, k in ((1, 1, 16, 4096, 4096), (2, 1, 16, 2048, 8192), (1, 1, 16, 8192, 2048),
                                (1, 1, 16, 16384, 4096), (1, 1, 96, 8192, 8192), (2, 1, 1024, 1024, 32768),
                                (1, 0, 16, 8192, 16384), (2, 0, 16, 4096, 16384), (0, 1, 16, 8192, 8192),
                                (0, 0, 512, 512, 65536), (1, 0, 8192, 8192, 8192), (0, 1, 2048, 2048, 16384)):
        s, cfg = splits_of(L, prec, rowb, m, n, k)
        assert s == 1 and cfg == L.pdgemm_pick_config(prec, m, n, k), (prec, rowb, m, n, k)
    assert splits_of(L, 3, 0, 64, 64, 64) == (-1, -1)
    assert L.pdgemm_pick_splits(1, 1, 64, 8192, 8192, None) == 2


def test_pick_splits_invariants(sklib):
    L = sklib
    info = {}
    for cfg in range(L.pdgemm_num_configs()):
        vals = [ctypes.c_int() for _ in range(5)]
        L.pdgemm_config_info(cfg, *[ctypes.byref(v) for v in vals])
        info[cfg] = tuple(v.value for v in vals)[:2]
    seen = set()
    for prec in range(3):
        for rowb in (0, 1):
            for m in (1, 16, 48, 64, 65, 96, 200, 512, 1024, 4096):
                for n in (64, 500, 2048, 4096, 8192, 16384):
                    for k in (0, 256, 2048, 4096, 8192, 16384, 65536, 131070):
                        s, cfg = splits_of(L, prec, rowb, m, n, k)
                        if s == 1:
                            assert cfg == L.pdgemm_pick_config(prec, m, n, k)
                            continue
                        seen.add(s)
                        bm, bn = info[cfg]
                        tiles = -(-m // bm) * -(-n // bn)
                        assert cfg in (2, 5) and s in (2, 4, 8), (prec, rowb, m, n, k, s, cfg)
                        assert tiles * s <= 256
                        if prec == 0:
                            assert s == 2 and rowb and k >= 16384
                        else:   # the largest split with at most 256 workgroups
                            assert s == 8 or tiles * s * 2 > 256
                            assert k // s >= (2048 if rowb else 4096)
                        if cfg == 5:
                            assert prec != 0 and m > 64
    assert seen == {2, 4, 8}


def test_splitk_errors_before_any_hip_call(sklib):
    L = sklib
    c = codes()
    n = L.pdgemm_num_configs()
    def sk(prec=1, cfg=2, rowb=0, splits=2, M=64, N=64, K=4096, A=PA, lda=None, B=PB, ldb=None):
        lda = K if lda is None else lda
        ldb = (N if rowb else K) if ldb is None else ldb
        return L.pdgemm_gemm_splitk_cfg(prec, cfg, rowb, splits, M, N, K, A, lda, B, ldb, PC, N, None)
    for cfg in (-1, 0, 1, 3, 4, 6, 7, 8, 9, n):   # only the tiles without an in-workgroup K split, 2 and 5
        assert sk(cfg=cfg) == c["PDGEMM_EINVAL_CFG"], cfg
    assert sk(prec=3) == c["PDGEMM_EINVAL_CFG"]
    assert sk(splits=0) == c["PDGEMM_EINVAL_CFG"]
    assert sk(prec=0, splits=3) == c["PDGEMM_EINVAL_CFG"]          # FP16: at most two ranges
    assert sk(prec=0, splits=4, rowb=1) == c["PDGEMM_EINVAL_CFG"]
    assert sk(lda=4000) == c["PDGEMM_EINVAL_LD"]
    assert sk(rowb=1, ldb=32) == c["PDGEMM_EINVAL_LD"]
    assert sk(B=None) == c["PDGEMM_ENULL"]
    assert sk(A=PA + 8) == c["PDGEMM_EALIGN"]
    assert sk(prec=2, K=4095, lda=4096, ldb=4096) == c["PDGEMM_EINVAL_I4"]
    assert sk(M=-1) == c["PDGEMM_EINVAL_DIM"]
    assert sk(M=0) == 0 and sk(N=0, rowb=0) == 0


@pytest.fixture(scope="module")
def wslib(lib):
    i64, p, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    for name in ("gemm_i4_ws", "gemm_i4_rowb_ws"):
        getattr(lib, name).argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p]
        getattr(lib, name).restype = i
    lib.gemm_i4_dequant_ws.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p, i64, p]
    lib.gemm_i4_dequant_ws.restype = i
    lib.pdgemm_i4_f6_cfg.argtypes = [i, i, i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p, i64, p]
    lib.pdgemm_i4_f6_cfg.restype = i
    for name in ("pdgemm_i4_workspace_size", "pdgemm_i4_f6_workspace_bytes"):
        getattr(lib, name).argtypes = [i64, i64, i64]
        getattr(lib, name).restype = i64
    lib.pdgemm_i4_f6_pick.argtypes = [i64, i64, i64]
    lib.pdgemm_i4_f6_pick.restype = i
    lib.pdgemm_i4_f6_image_bytes.argtypes = [i64, i64]
    lib.pdgemm_i4_f6_image_bytes.restype = i64
    lib.pdgemm_i4_f6_pack.argtypes = [i64, i64, p, i64, i, p, i64, p]
    lib.pdgemm_i4_f6_pack.restype = i
    lib.gemm_i4_packed_b.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, p]
    lib.gemm_i4_packed_b.restype = i
    lib.gemm_i4_dequant_packed_b.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p, i64, p]
    lib.gemm_i4_dequant_packed_b.restype = i
    lib.pdgemm_i4_packed_b_cfg.argtypes = [i, i64, i64, i64, p, i64, p, i64, p, p, p, i64, i, p, i64, p]
    lib.pdgemm_i4_packed_b_cfg.restype = i
    return lib


def f6_bytes(M, N, K):
    """The workspace size rule the header states, restated: two images of
    32-row groups x 128-value K blocks (padded to a multiple of 3) of 3072
    bytes, B's starting at the next multiple of 256 bytes after A's."""
    cd = lambda a, b: -(-a // b)
    blocks = cd(cd(K, 128), 3) * 3
    img = lambda rows: cd(rows, 32) * blocks * 3072
    return cd(img(M), 256) * 256 + img(N)


def test_workspace_sizes(wslib):
    L = wslib
    for M, N, K in ((8192, 8192, 8192), (4096, 4096, 4096), (4000, 3000, 1030), (5000, 777, 131070)):
        assert L.pdgemm_i4_f6_workspace_bytes(M, N, K) == f6_bytes(M, N, K)
        want = f6_bytes(M, N, K) if L.pdgemm_i4_f6_pick(M, N, K) >= 0 else 0
        assert L.pdgemm_i4_workspace_size(M, N, K) == want
    # the FP6 path takes large products only; small ones need no workspace
    assert L.pdgemm_i4_f6_pick(8192, 8192, 8192) == 0 and L.pdgemm_i4_f6_pick(4096, 4096, 4096) == 0
    for shape in ((2048, 2048, 2048), (64, 8192, 8192), (8192, 8192, 512), (0, 10, 10)):
        assert L.pdgemm_i4_f6_pick(*shape) == -1 and L.pdgemm_i4_workspace_size(*shape) == 0
    assert L.pdgemm_i4_workspace_size(-1, 5, 5) == 0


def test_workspace_errors_before_any_hip_call(wslib):
    L, c = wslib, codes()
    M = N = K = 4096
    need = L.pdgemm_i4_workspace_size(M, N, K)
    A, B, C, ws = 0x10000, 0x20000, 0x30000, 0x100000
    args = lambda w, n: (M, N, K, A, K, B, K, C, N, w, n, None)
    assert L.gemm_i4_ws(*args(None, need)) == c["PDGEMM_ENULL"]
    assert L.gemm_i4_ws(*args(ws, need - 1)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_ws(*args(ws + 8, need)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_ws(*args(ws, -5)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_rowb_ws(*args(ws, need - 16)) == c["PDGEMM_EWORKSPACE"]
    # argument errors come first, as for gemm_i4
    assert L.gemm_i4_ws(M, N, K + 1, A, K + 1, B, K + 1, C, N, ws, need, None) == c["PDGEMM_EINVAL_I4"]
    assert L.gemm_i4_ws(M, N, K, A, K, B, K, C, N - 1, ws, need, None) == c["PDGEMM_EINVAL_LD"]
    assert L.gemm_i4_dequant_ws(M, N, K, A, K, B, K, None, None, C, N, 0, ws, need, None) == c["PDGEMM_ENULL"]
    assert L.gemm_i4_dequant_ws(M, N, K, A, K, B, K, 0x40000, 0x50000, C, N, 1, ws, 16, None) == \
        c["PDGEMM_EWORKSPACE"]
    # the explicit FP6 tiles: unknown tile, then the workspace rule for any shape
    assert L.pdgemm_i4_f6_cfg(7, 0, M, N, K, A, K, B, K, None, None, C, N, 0, ws, need, None) == \
        c["PDGEMM_EINVAL_CFG"]
    small = f6_bytes(300, 200, 1030)
    assert L.pdgemm_i4_f6_cfg(1, 0, 300, 200, 1030, A, 1056, B, 1056, None, None, C, 200, 0, ws, small - 1,
                              None) == c["PDGEMM_EWORKSPACE"]
    assert L.pdgemm_strerror(c["PDGEMM_EWORKSPACE"]).decode().startswith("workspace")


def test_image_sizes(wslib):
    # one operand's image: 32-row groups x 128-value K blocks (padded to a multiple of 3) of 3072
    # bytes; the workspace holds A's image, then B's at the next multiple of 256 bytes
    L = wslib
    cd = lambda a, b: -(-a // b)
    for rows, K in ((1, 2), (31, 130), (8192, 8192), (5000, 131070)):
        assert L.pdgemm_i4_f6_image_bytes(rows, K) == cd(rows, 32) * cd(cd(K, 128), 3) * 3 * 3072
    for M, N, K in ((8192, 8192, 8192), (4000, 3000, 1030)):
        a = L.pdgemm_i4_f6_image_bytes(M, K)
        assert L.pdgemm_i4_f6_workspace_bytes(M, N, K) == cd(a, 256) * 256 + L.pdgemm_i4_f6_image_bytes(N, K)
    assert L.pdgemm_i4_f6_image_bytes(-1, 8) == 0 and L.pdgemm_i4_f6_image_bytes(8, 0) == 0


def test_packed_b_errors_before_any_hip_call(wslib):
    L, c = wslib, codes()
    M, N, K = 1024, 8192, 8192
    A, B, C, img, ws = 0x10000, 0x20000, 0x30000, 0x100000, 0x200000
    nb, na = L.pdgemm_i4_f6_image_bytes(N, K), L.pdgemm_i4_f6_image_bytes(M, K)
    # pack: argument rules as for the operand of a GEMM, then the image
    assert L.pdgemm_i4_f6_pack(-1, K, B, K, 0, img, nb, None) == c["PDGEMM_EINVAL_DIM"]
    assert L.pdgemm_i4_f6_pack(N, 131072, B, 131072, 0, img, nb, None) == c["PDGEMM_EINVAL_DIM"]
    assert L.pdgemm_i4_f6_pack(N, K, B, K - 2, 0, img, nb, None) == c["PDGEMM_EINVAL_LD"]
    assert L.pdgemm_i4_f6_pack(N, K, B, N - 2, 1, img, nb, None) == c["PDGEMM_EINVAL_LD"]
    assert L.pdgemm_i4_f6_pack(N, K + 1, B, K + 2, 0, img, nb, None) == c["PDGEMM_EINVAL_I4"]
    assert L.pdgemm_i4_f6_pack(N, K, None, K, 0, img, nb, None) == c["PDGEMM_ENULL"]
    assert L.pdgemm_i4_f6_pack(N, K, B, K, 0, None, nb, None) == c["PDGEMM_ENULL"]
    assert L.pdgemm_i4_f6_pack(N, K, B + 8, K, 0, img, nb, None) == c["PDGEMM_EALIGN"]
    assert L.pdgemm_i4_f6_pack(N, K, B, K + 2, 0, img, nb, None) == c["PDGEMM_EALIGN"]
    assert L.pdgemm_i4_f6_pack(N, K, B, K, 0, img, nb - 1, None) == c["PDGEMM_EWORKSPACE"]
    assert L.pdgemm_i4_f6_pack(N, K, B, K, 0, img + 8, nb, None) == c["PDGEMM_EWORKSPACE"]
    assert L.pdgemm_i4_f6_pack(0, K, None, K, 0, None, 0, None) == c["PDGEMM_OK"]   # an empty image
    # the GEMM from A and B's image
    args = lambda ib, nbb, w, nw: (M, N, K, A, K, ib, nbb, C, N, w, nw, None)
    assert L.gemm_i4_packed_b(*args(img, nb, None, na)) == c["PDGEMM_ENULL"]
    assert L.gemm_i4_packed_b(*args(None, nb, ws, na)) == c["PDGEMM_ENULL"]
    assert L.gemm_i4_packed_b(*args(img, nb - 1, ws, na)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_packed_b(*args(img, nb, ws, na - 1)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_packed_b(*args(img + 8, nb, ws, na)) == c["PDGEMM_EWORKSPACE"]
    assert L.gemm_i4_packed_b(M, N, K, A, K - 2, img, nb, C, N, ws, na, None) == c["PDGEMM_EINVAL_LD"]
    assert L.gemm_i4_packed_b(M, N, K, A, K, img, nb, C, N - 1, ws, na, None) == c["PDGEMM_EINVAL_LD"]
    assert L.gemm_i4_packed_b(M, N, K + 1, A, K + 2, img, nb, C, N, ws, na, None) == c["PDGEMM_EINVAL_I4"]
    assert L.gemm_i4_packed_b(M, N, K, A + 8, K, img, nb, C, N, ws, na, None) == c["PDGEMM_EALIGN"]
    assert L.gemm_i4_packed_b(0, N, K, None, K, None, 0, None, N, None, 0, None) == c["PDGEMM_OK"]
    assert L.gemm_i4_dequant_packed_b(M, N, K, A, K, img, nb, None, None, C, N, 0, ws, na, None) == \
        c["PDGEMM_ENULL"]
    assert L.pdgemm_i4_packed_b_cfg(-1, M, N, K, A, K, img, nb, None, None, C, N, 0, ws, na, None) == \
        c["PDGEMM_EINVAL_CFG"]
    assert L.pdgemm_i4_packed_b_cfg(2, M, N, K, A, K, img, nb, None, None, C, N, 0, ws, na, None) == \
        c["PDGEMM_EINVAL_CFG"]
