"""CPU checks of the kernel's LDS layout and block order rules (restated here
from their definitions in the kernel source)."""
from __future__ import annotations

import itertools


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


def remap(bid, nb, tiles_m, tiles_n, band):
    q, r = nb >> 3, nb & 7
    xcd, loc = bid & 7, bid >> 3
    i = xcd * (q + 1) + loc if xcd < r else r * (q + 1) + (xcd - r) * q + loc
    b = i // (band * tiles_n)
    first = b * band
    rows = min(tiles_m - first, band)
    inb = i - b * band * tiles_n
    return first + inb % rows, inb // rows


def test_block_remap_is_a_bijection():
    for tm, tn, band in itertools.product(range(1, 34), range(1, 34), (1, 4, 8)):
        nb = tm * tn
        seen = {remap(b, nb, tm, tn, band) for b in range(nb)}
        assert len(seen) == nb
        assert all(0 <= m < tm and 0 <= n < tn for m, n in seen)


def test_xcd_locality_at_8192():
    # N = 8192 with 256x256 tiles: the 32 workgroups first resident on XCD 0 cover 4 x 8 tiles
    tiles = 32
    first = [remap(b, tiles * tiles, tiles, tiles, 4) for b in range(0, 8 * 32, 8)]
    assert len({m for m, _ in first}) == 4 and len({n for _, n in first}) == 8
