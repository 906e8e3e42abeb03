"""CPU checks of the kernel's LDS layout and block order rules (restated here
from their definitions in the kernel source)."""
from __future__ import annotations

import itertools

import pytest


def swizzle(r: int) -> int:
    # LDS position of logical 16-byte chunk c of 64-byte row r is c ^ swizzle(r)
    return ((r >> 1) & 3) ^ ((r >> 3) & 1)


def test_swizzle_is_a_permutation_of_each_row():
    for r in range(1024):
        assert sorted(c ^ swizzle(r) for c in range(4)) == [0, 1, 2, 3]


def test_fragment_reads_are_bank_conflict_free():
    # a quarter-wave reads 16 consecutive rows (from a multiple of 16) at one logical chunk
    for base in range(0, 1024, 16):
        rows = [base + i for i in range(16)]
        for c in range(4):
            # 64 banks of 4 bytes: row r, position p covers banks 16*(r%4) + 4p .. +3
            assert len({16 * (r % 4) + 4 * (c ^ swizzle(r)) for r in rows}) == 16
            # 32 banks: each group of 8 lanes must cover distinct 16-byte bank groups
            for o in (0, 8):
                assert len({16 * (r % 2) + 4 * (c ^ swizzle(r)) for r in rows[o:o + 8]}) == 8



def swizzle8(r: int) -> int:
    # rows of 128 bytes (whole-line staging): logical chunk c of row r sits at c ^ swizzle8(r)
    return (r & 7) ^ ((r >> 3) & 1)


def test_line_swizzle_is_a_permutation_of_each_row():
    for r in range(1024):
        assert sorted(c ^ swizzle8(r) for c in range(8)) == list(range(8))


def test_line_fragment_reads_are_bank_conflict_free():
    # a quarter-wave reads 16 consecutive rows (from a multiple of 16) at one logical chunk;
    # a 128-byte row r at position p covers banks 32*(r%2) + 4p .. +3 of 64
    for base in range(0, 1024, 16):
        rows = [base + i for i in range(16)]
        for c in range(8):
            assert len({32 * (r % 2) + 4 * (c ^ swizzle8(r)) for r in rows}) == 16
            # 32 banks: 8 consecutive rows at distinct positions
            for o in (0, 8):
                assert len({c ^ swizzle8(r) for r in rows[o:o + 8]}) == 8


def swizzle16(r: int) -> int:
    # rows of 128 bytes in the FP16 16 x 16 MFMA tile: logical chunk c of row r sits at c ^ swizzle16(r)
    return ((r ^ (r >> 1)) & 1) | ((r >> 2) & 2) | (r & 4)


# ds_read_b128 serves a wave in four phases of 16 lanes: lanes 8p .. 8p+7 with 32+8p .. 32+8p+7
# (the grouping under which rocprofv3's SQ_LDS_BANK_CONFLICT reads 4 extra cycles per read for the
# 16 x 16 reads on swizzle8, and none for the 32 x 32 reads on swizzle8, as measured)
READ_PHASES = [list(range(8 * p, 8 * p + 8)) + list(range(32 + 8 * p, 40 + 8 * p)) for p in range(4)]


def extra_cycles(rowchunk, swz, phases=READ_PHASES):
    """Conflict cycles of one ds_read_b128 with 128-byte rows: lane l reads logical chunk c of
    row r (rowchunk(l) = (r, c)); row r at position p covers 16-byte bank group 8 (r % 2) + p."""
    extra = 0
    for ph in phases:
        groups = {}
        for lane in ph:
            r, c = rowchunk(lane)
            g = 8 * (r % 2) + (c ^ swz(r))
            groups[g] = groups.get(g, 0) + 1
        extra += max(groups.values()) - 1
    return extra


def test_read_phase_model_matches_the_counters():
    for base in range(0, 512, 32):
        for q in range(4):   # the 32 x 32 reads of the whole-line tiles: no conflicts
            assert extra_cycles(lambda l: (base + l % 32, 2 * q + l // 32), swizzle8) == 0
    for q in (0, 1):         # the 16 x 16 reads on swizzle8: 4 extra cycles, as counted
        assert extra_cycles(lambda l: (l % 16, 4 * q + l // 16), swizzle8) == 4


def test_mf16_fragment_reads():
    # The FP16 256 x 256 tile on 16 x 16 MFMAs: in k-step q (0, 1) of a 128-byte stage row,
    # lane l of a 16-row block reads row l%16 at logical chunk 4q + l//16, i.e. f16 values
    # 32q + 8(l//16) .. +7, the 8 values of K the MFMA expects in that lane.
    for base in range(0, 512, 16):
        covered = {}
        for q in (0, 1):
            rc = lambda l: (base + l % 16, 4 * q + l // 16)
            assert extra_cycles(rc, swizzle16) == 0
            # also conflict-free if the phases were plain quarter-waves
            assert extra_cycles(rc, swizzle16, [list(range(16 * p, 16 * p + 16)) for p in range(4)]) == 0
            for lane in range(64):
                r, c = rc(lane)
                assert c * 8 == 32 * q + 8 * (lane // 16)   # first f16 value of K in the lane
                covered[(r, c)] = covered.get((r, c), 0) + 1
        # the two k-steps read every 16-byte chunk of the 16 rows exactly once
        assert covered == {(base + i, c): 1 for i in range(16) for c in range(8)}
    # the swizzle permutes the chunks of every row (DMA writes and reads agree)
    for r in range(512):
        assert sorted(c ^ swizzle16(r) for c in range(8)) == list(range(8))


def bswizzle16(prec: str, bn: int, r: int) -> int:
    # row-major B in the 16 x 16 tile: logical chunk c of B row r sits at c ^ bswizzle16(r)
    if prec == "f16":
        return 2 * ((r & 3) | ((((r >> 3) ^ (r >> 4)) & 1) << 2))
    if bn == 256:
        return (r & 7) | ((((r >> 4) ^ (r >> 5)) & 1) << 3)
    return ((r >> 1) & 3) | ((((r >> 4) ^ (r >> 5)) & 1) << 2)


@pytest.mark.parametrize("prec", ["f16", "i8"])
@pytest.mark.parametrize("bn", [256, 128])
def test_mf16_rowmajor_b_reads(prec, bn):
    # transposing reads (ds_read_b64_tr_b16 / _b8): lane i of 16-lane group g addresses row
    # 2 kR g + kR t + i // kQ of the k-step, bytes 8 (i % kQ) of the group's 16 columns, and
    # receives kR values of column i; the stage's B part holds rows of kCpr chunks
    es, kr = (2, 4) if prec == "f16" else (1, 8)
    kq = 16 // kr
    kcpr = bn * es // 16
    krows = 32 if prec == "f16" else 64          # rows of B per 64-byte k-step
    assert 2 * krows * kcpr == 8 * bn            # the B part of a stage: bn rows of 128 bytes
    for wn0 in range(0, bn, 64):
        for j in range(4):
            for q in (0, 1):
                for t in (0, 1):
                    slots = {}
                    for lane in range(64):
                        g, i = lane // 16, lane % 16
                        row = q * krows + g * 2 * kr + t * kr + i // kq
                        col_bytes = (wn0 + 16 * j) * es + 8 * (i % kq)
                        # the lane's swizzle does not depend on q or t (the kernel hoists it)
                        assert bswizzle16(prec, bn, row) == bswizzle16(prec, bn, g * 2 * kr + i // kq)
                        pos = (col_bytes >> 4) ^ bswizzle16(prec, bn, row)
                        assert 0 <= pos < kcpr
                        slots[lane] = (row * kcpr + pos) * 16 + (col_bytes & 15)
                        # the DMA put logical chunk (col_bytes >> 4) of this row at that position
                        assert (pos ^ bswizzle16(prec, bn, row)) == col_bytes >> 4
                    # 8-byte reads, 256 bytes per cycle: either pairing of 16-lane groups per cycle
                    # touches 16 distinct 16-byte bank groups with two lanes each
                    for pairing in (((0, 1), (2, 3)), ((0, 2), (1, 3))):
                        for pair in pairing:
                            lanes = [l for l in range(64) if l // 16 in pair]
                            groups = {}
                            for l in lanes:
                                bg = (slots[l] // 16) % 16
                                groups.setdefault(bg, set()).add(slots[l] // 16)
                            assert len(groups) == 16 and all(len(v) == 1 for v in groups.values())


def permlane16_swap(x, y):
    # v_permlane16_swap_b32 x, y: the odd 16-lane rows of x trade places with the even ones of y
    rows = lambda v: [v[16 * k:16 * k + 16] for k in range(4)]
    xr, yr = rows(x), rows(y)
    return xr[0] + yr[0] + xr[2] + yr[2], xr[1] + yr[1] + xr[3] + yr[3]


@pytest.mark.parametrize("fm", [8, 4, 2])
def test_mf16_result_layout_covers_the_wave_tile(fm):
    # register e of lane l in block (i, j): row 16i + 4(l//16) + e, column 16j + l%16; the
    # epilogue swaps blocks 2h and 2h+1 and stores the first result at row 16i + e + 8(l//32),
    # the second 4 rows below, column 32h + l%32: each element of the 16 fm x 64 wave tile
    # (128, 64 or 32 rows) once, each store two whole 128-byte rows
    stored = {}
    for i in range(fm):
        for e in range(4):
            for h in range(2):
                held = [[(16 * i + 4 * (l // 16) + e, 16 * j + l % 16) for l in range(64)] for j in (2 * h, 2 * h + 1)]
                x, y = permlane16_swap(held[0], held[1])
                for k, reg in enumerate((x, y)):
                    for l in range(64):
                        want = (16 * i + e + 4 * k + 8 * (l // 32), 32 * h + l % 32)
                        assert reg[l] == want
                        stored[want] = stored.get(want, 0) + 1
    assert stored == {(r, c): 1 for r in range(16 * fm) for c in range(64)}


@pytest.mark.parametrize("bm,bn,waves", [(256, 256, 8), (128, 128, 8), (64, 64, 4), (256, 128, 8), (128, 64, 4),
                                         (32, 32, 1), (64, 32, 1)])
def test_line_dma_fills_every_row_once(bm, bn, waves):
    # instruction j of wave w writes LDS rows (j*waves + w)*8 .. +7, lane l to row l/8 at
    # position l%8, fetching logical chunk (l%8) ^ swizzle8(row) of that row: every
    # (row, position) is written once, with the chunk the fragment reads expect there
    rows = bm + bn
    per_wave = rows // 8 // waves
    seen = {}
    for w in range(waves):
        for j in range(per_wave):
            for lane in range(64):
                r = (j * waves + w) * 8 + lane // 8
                pos = lane % 8
                assert (r, pos) not in seen
                seen[(r, pos)] = pos ^ swizzle8(r)
    assert len(seen) == rows * 8
    for r in range(rows):
        for c in range(8):
            assert seen[(r, c ^ swizzle8(r))] == c


def remap(bid, nb, tiles_m, tiles_n, band):
    q, r = nb >> 3, nb & 7
    xcd, loc = bid & 7, bid >> 3
    i = xcd * (q + 1) + loc if xcd < r else r * (q + 1) + (xcd - r) * q + loc
    b = i // (band * tiles_n)
    first = b * band
    rows = min(tiles_m - first, band)
    inb = i - b * band * tiles_n
    return first + inb % rows, inb // rows


def tile_order(bid, tiles_m, tiles_n, band, windows=True):
    """tile_of: 16 x 16 windows of tiles where the large tiles (band 4) fill whole windows, else bands."""
    if windows and band == 4 and (tiles_m | tiles_n) % 16 == 0:
        x, loc = bid & 7, bid >> 3
        w, k = loc >> 5, loc & 31
        wcols = tiles_n >> 4
        wm, wi = divmod(w, wcols)
        wn = wcols - 1 - wi if wm & 1 else wi
        return wm * 16 + (x & 3) * 4 + (k & 3), wn * 16 + (x >> 2) * 8 + (k >> 2)
    return remap(bid, tiles_m * tiles_n, tiles_m, tiles_n, band)


def test_block_remap_is_a_bijection():
    for tm, tn, band in itertools.product(range(1, 34), range(1, 34), (1, 4, 8)):
        nb = tm * tn
        seen = {remap(b, nb, tm, tn, band) for b in range(nb)}
        assert len(seen) == nb
        assert all(0 <= m < tm and 0 <= n < tn for m, n in seen)


def test_window_order_is_a_bijection():
    for tm, tn in itertools.product((16, 32, 48, 64, 80), repeat=2):
        nb = tm * tn
        seen = {tile_order(b, tm, tn, 4) for b in range(nb)}
        assert len(seen) == nb
        assert all(0 <= m < tm and 0 <= n < tn for m, n in seen)
    # grids that are not whole windows keep the band order
    for tm, tn in ((16, 24), (33, 32), (8, 64)):
        assert [tile_order(b, tm, tn, 4) for b in range(tm * tn)] == \
            [remap(b, tm * tn, tm, tn, 4) for b in range(tm * tn)]


def test_xcd_locality_at_8192():
    # N = 8192 with 256x256 tiles: the 32 workgroups first resident on each XCD cover 4 x 8 tiles,
    # in both orders
    tiles = 32
    for windows in (False, True):
        for x in range(8):
            first = [tile_order(b, tiles, tiles, 4, windows) for b in range(x, 8 * 32, 8)]
            assert len({m for m, _ in first}) == 4 and len({n for _, n in first}) == 8


def test_window_rounds_at_8192():
    # each round of 256 workgroups covers one 16 x 16 window: 16 panels of A and 16 of B (the band
    # order: all 32 of A and 8 of B), and each window shares its rows or columns with the one before
    tiles = 32
    rounds = [[tile_order(b, tiles, tiles, 4) for b in range(256 * r, 256 * (r + 1))] for r in range(4)]
    bands = [[remap(b, tiles * tiles, tiles, tiles, 4) for b in range(256 * r, 256 * (r + 1))] for r in range(4)]
    for r in range(4):
        assert len({m for m, _ in rounds[r]}) == 16 and len({n for _, n in rounds[r]}) == 16
        assert len({m for m, _ in bands[r]}) == 32 and len({n for _, n in bands[r]}) == 8
    for r in range(1, 4):
        rows = lambda t: {m for m, _ in t}
        cols = lambda t: {n for _, n in t}
        assert rows(rounds[r]) == rows(rounds[r - 1]) or cols(rounds[r]) == cols(rounds[r - 1])


# --------------------------------------------------------------------------
# Row-major B: DMA placement, transposing reads and banks (restated from the
# kernel source; the read semantics are those measured for gfx950's
# ds_read_b64_tr_b16 / _b8 / _b4: in a 16-lane group, result element e of
# lane i comes from the 8 bytes addressed by source lane j at element p, with
# (j, p) = (i//4 + 4e, i%4) for b16, (i//8 + 2e, i%8) for b8, (e, i) for b4).


ROWB = {  # precision: (rows per K tile, rows per read R, elements per 16-byte chunk, bits)
    "f16": (32, 4, 8, 16),
    "i8": (64, 8, 16, 8),
    "i4": (128, 16, 32, 4),
}
# the tiles without K split, and one K slice of the K-split tiles (32 x 32, 64 x 32)
CONFIGS = [(256, 256, 128, 128), (128, 128, 64, 64), (64, 64, 32, 32), (256, 128, 128, 64), (128, 64, 64, 32),
           (32, 32, 32, 32), (64, 32, 64, 32)]


def bswizzle(prec, bn, r):
    _, R, epc, _ = ROWB[prec]
    Q = 16 // R
    cpr = bn // epc
    v = 1 if cpr >= 16 else 16 // cpr
    span = min(cpr, 16) // Q
    return Q * ((r // v) % span)


def tr_source(prec, i, e):
    """(source lane, element within its 8 bytes) of result element e of group lane i."""
    if prec == "f16":
        return i // 4 + 4 * e, i % 4
    if prec == "i8":
        return i // 8 + 2 * e, i % 8
    return e, i


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=["256", "128", "64", "256x128", "128x64", "ks32x32", "ks64x32"])
def test_rowmajor_b_layout(prec, cfg):
    BM, BN, WM, WN = cfg
    krows, R, epc, bits = ROWB[prec]
    Q = 16 // R
    cpr = BN // epc
    NW = (BM // WM) * (BN // WN)
    kdma = (BM + BN) // 16 // NW
    kdma_a = BM // 16 // NW
    # DMA: every LDS chunk slot of the B part receives one distinct (row, chunk) of the tile
    slot_src = {}
    for wave in range(NW):
        for j in range(kdma_a, kdma):
            for lane in range(64):
                cr = (j * NW + wave) * 16 + lane // 4
                f = (cr - BM) * 4 + lane % 4
                krow, pos = f // cpr, f % cpr
                g = pos ^ bswizzle(prec, BN, krow)
                assert 0 <= krow < krows and 0 <= g < cpr
                slot_src[f] = (krow, g)
    assert sorted(slot_src) == list(range(krows * cpr))
    assert len(set(slot_src.values())) == krows * cpr

    def element_at(byte_addr, elem):
        """(k, n) of element `elem` of the 8 bytes at LDS byte address byte_addr of the B part."""
        f, inb = byte_addr // 16, byte_addr % 16
        krow, g = slot_src[f]
        col_byte = g * 16 + inb
        return krow, col_byte * 8 // bits + elem

    steprows = krows // 2
    for wave in range(NW):
        wn0 = (wave % (BN // WN)) * WN
        for s in range(2):
            for jj in range(WN // 32):
                lane_bytes = {}   # LDS byte address of each lane, per read
                for r in range(2):
                    addrs = []
                    for lane in range(64):
                        i, grp, half = lane % 16, (lane >> 4) & 1, lane >> 5
                        col_bytes = (wn0 + jj * 32) * bits // 8 + (16 * grp) * bits // 8 + 8 * (i % Q)
                        krow = s * steprows + half * (steprows // 2) + r * R + i // Q
                        pos = (col_bytes >> 4) ^ bswizzle(prec, BN, krow)
                        addr = (krow * cpr + pos) * 16 + (col_bytes & 15)
                        assert 0 <= addr and addr + 8 <= krows * cpr * 16
                        addrs.append(addr)
                    lane_bytes[r] = addrs
                    # banks: each half-wave touches 64 distinct 4-byte banks
                    for hw in (0, 32):
                        banks = [(a // 4 + w) % 64 for a in addrs[hw:hw + 32] for w in (0, 1)]
                        assert len(set(banks)) == 64, (prec, cfg, s, jj, r)
                # the fragment each lane assembles: K-contiguous values of its own column
                per_read = 64 // bits     # elements per 8 bytes
                for lane in range(64):
                    grp0 = lane - lane % 16
                    i, half = lane % 16, lane >> 5
                    for r in range(2):
                        for e in range(per_read):
                            src, p = tr_source(prec, i, e)
                            k, n = element_at(lane_bytes[r][grp0 + src], p)
                            want_k = s * steprows + half * (steprows // 2) + r * per_read + e
                            assert (k, n) == (want_k, wn0 + jj * 32 + lane % 32), (prec, cfg, lane, r, e)


# the tiles without K split (4 or 8 waves), and one K slice of the K-split tiles (a slice is
# staged and read by one wave, as a one-wave tile)
LINE_CONFIGS = [(256, 256, 128, 64), (128, 128, 32, 64), (64, 64, 32, 32), (256, 128, 64, 64), (128, 64, 64, 32),
                (32, 32, 32, 32), (64, 32, 64, 32)]


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("cfg", LINE_CONFIGS, ids=["256", "128", "64", "256x128", "128x64", "ks32x32", "ks64x32"])
def test_rowmajor_b_line_layout(prec, cfg):
    # Whole-line stages hold two K tiles: the B part is 2 * krows rows of B.  DMA
    # instruction j of wave w fills 1 KB block j*NW + w of the stage (lane l: chunk l of
    # the block); blocks past the A part hold flat chunks f of the B part, row f // cpr,
    # position f % cpr, fetching chunk position ^ bswizzle(row).  The transposing reads
    # of k-steps 0..3 must find K-contiguous values of their own column, conflict-free.
    BM, BN, WM, WN = cfg
    krows, R, epc, bits = ROWB[prec]
    Q = 16 // R
    cpr = BN // epc
    NW = (BM // WM) * (BN // WN)
    rows = 2 * krows
    blocks = (BM + BN) // 8
    slot_src = {}
    for wave in range(NW):
        for j in range(blocks // NW):
            b = j * NW + wave
            if b < BM // 8:
                continue
            for lane in range(64):
                f = (b - BM // 8) * 64 + lane
                krow, pos = f // cpr, f % cpr
                g = pos ^ bswizzle(prec, BN, krow)
                assert 0 <= krow < rows and 0 <= g < cpr
                slot_src[f] = (krow, g)
    assert sorted(slot_src) == list(range(rows * cpr))
    assert len(set(slot_src.values())) == rows * cpr

    steprows = krows // 2
    per_read = 64 // bits
    for wave in range(NW):
        wn0 = (wave % (BN // WN)) * WN
        for s in range(4):
            for jj in range(WN // 32):
                lane_bytes = {}
                for r in range(2):
                    addrs = []
                    for lane in range(64):
                        i, grp, half = lane % 16, (lane >> 4) & 1, lane >> 5
                        col_bytes = (wn0 + jj * 32) * bits // 8 + (16 * grp) * bits // 8 + 8 * (i % Q)
                        krow = s * steprows + half * (steprows // 2) + r * R + i // Q
                        pos = (col_bytes >> 4) ^ bswizzle(prec, BN, krow)
                        addr = (krow * cpr + pos) * 16 + (col_bytes & 15)
                        assert 0 <= addr and addr + 8 <= rows * cpr * 16
                        addrs.append(addr)
                    lane_bytes[r] = addrs
                    for hw in (0, 32):
                        banks = [(a // 4 + w) % 64 for a in addrs[hw:hw + 32] for w in (0, 1)]
                        assert len(set(banks)) == 64, (prec, cfg, s, jj, r)
                for lane in range(64):
                    grp0 = lane - lane % 16
                    i, half = lane % 16, lane >> 5
                    for r in range(2):
                        for e in range(per_read):
                            src, p = tr_source(prec, i, e)
                            f, inb = lane_bytes[r][grp0 + src] // 16, lane_bytes[r][grp0 + src] % 16
                            krow, g = slot_src[f]
                            k, n = krow, (g * 16 + inb) * 8 // bits + p
                            want_k = s * steprows + half * (steprows // 2) + r * per_read + e
                            assert (k, n) == (want_k, wn0 + jj * 32 + lane % 32), (prec, cfg, lane, r, e)


# Tiles (block rows, block columns, K split, whole-line stages) as the kernel's
# configuration table defines them; the 32 x 32 K-split tile stages 64-byte K
# tiles, every other tile whole 128-byte lines.
TILES = [(256, 256, 1, True), (128, 128, 1, True), (64, 64, 1, True), (32, 32, 4, False),
         (256, 128, 1, True), (128, 64, 1, True), (64, 32, 4, True), (128, 128, 1, True),
         (256, 256, 1, True), (64, 64, 4, True), (256, 256, 1, True)]
MAX_ROW_BYTES = 1 << 22


def test_tile_table_matches_library():
    import precision_dense_gemm_amd as pd
    assert pd.num_configs() == len(TILES)
    for cfg, (bm, bn, ks, _) in enumerate(TILES):
        info = pd.config_info(cfg)
        assert (info["block_m"], info["block_n"]) == (bm, bn)
        assert info["threads"] == (bm // info["wave_m"]) * (bn // info["wave_n"]) * ks * 64


@pytest.mark.parametrize("prec", ["f16", "i8", "i4"])
@pytest.mark.parametrize("cfg", range(len(TILES)))
def test_operand_offsets_fit_32_bits(prec, cfg):
    # Every DMA lane forms a 32-bit offset from the base of a buffer resource
    # whose range is capped at 2^31 - 1 bytes: an offset beyond it would read
    # zeros, one beyond 2^32 would wrap.  At the largest rows the library
    # accepts (4 MiB), each resource must span fewer rows than 2^31 bytes hold.
    # A and a column-major B: one resource per tile of rows (BM or BN rows),
    # offsets up to (rows - 1) * ld + the last 16-byte chunk of a stage.
    # Row-major B: one resource per wave slice of a stage (K-split waves get a
    # base of their own), spanning the K rows of that slice: krows (64-byte
    # stages) or 2 * krows (whole lines).
    bm, bn, ks, line = TILES[cfg]
    krows = ROWB[prec][0]
    ld = MAX_ROW_BYTES
    stage_k = (128 if line else 64) * ks     # bytes of K per row per stage
    limit = 2 ** 31 - 1
    for rows in (bm, bn):
        assert (rows - 1) * ld + stage_k <= limit
    slice_rows = krows * (2 if line else 1)
    cpr_bytes = ld                            # a row of B: every chunk of it may be addressed
    assert (slice_rows - 1) * ld + cpr_bytes <= limit + 1
    assert slice_rows * ld <= 2 ** 30, "a slice of a row-major B stage spans at most 1 GiB"


# ---- INT4 on the FP6 cores ----

def e2m3_value(code: int) -> float:
    """The OCP e2m3 (FP6) value of a 6-bit code: sign, 2 exponent bits of bias 1, 3 mantissa bits;
    exponent 0 holds the subnormals m / 8."""
    sign = -1.0 if code & 0x20 else 1.0
    e, m = (code >> 3) & 3, code & 7
    return sign * (m / 8.0 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 1))


def test_int4_values_are_exact_e2m3_codes():
    # the code of v / 8 for an INT4 value v is sign << 5 | |v|: |v| = 0..7 are the
    # subnormals, |v| = 8 is exponent 1 with mantissa 0 (1.0)
    for v in range(-8, 8):
        code = (0x20 if v < 0 else 0) | abs(v)
        assert code < 64 and e2m3_value(code) == v / 8.0
    # and with block scales 2^3 on both operands, a product is the integer a * b
    for a in range(-8, 8):
        for b in range(-8, 8):
            ca, cb = (0x20 if a < 0 else 0) | abs(a), (0x20 if b < 0 else 0) | abs(b)
            assert e2m3_value(ca) * 8 * e2m3_value(cb) * 8 == a * b


def tswizzle(r: int) -> int:
    return (r >> 3) & 3


def test_fp6_tail_reads_are_bank_conflict_free():
    # the 32 lanes of a half-wave read one 8-byte slot of 32 consecutive rows of 32 bytes;
    # row r at position p covers the 4-byte banks 8 (r % 8) + 2 p and + 1 of 64
    for base in range(0, 512, 32):
        for c in range(4):
            banks = set()
            for r in range(base, base + 32):
                p = c ^ tswizzle(r)
                banks |= {(8 * (r % 8) + 2 * p) % 64, (8 * (r % 8) + 2 * p + 1) % 64}
            assert len(banks) == 64
    # and each row's four slots are a permutation of its positions
    for r in range(64):
        assert sorted(c ^ tswizzle(r) for c in range(4)) == [0, 1, 2, 3]
