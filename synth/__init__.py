"""Seeded synthetic operands for the multi-precision square GEMM.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's callers.  It holds no GEMM arithmetic: it only draws numbers and
lays them out in the operand formats the GEMM consumes.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  Stream element i (0-based) of a seed s is
mix(s + (i+1)*GAMMA) with the published GAMMA, multipliers and shifts.

Value mappings (the pages fix only the distributions; these are our readings):
  int8      top byte of the 64-bit draw, two's complement, uniform on [-128, 127]
  int4      (draw >> 60) - 8, uniform on [-8, 7]
  U[-1, 1)  2*u - 1 with u = (draw >> 11) * 2**-53, then rounded to binary16
            (round-to-nearest-even; 1 - 2**-12 and above round to 1.0)
  N(0, 1)   Box-Muller on consecutive draws (u1 in (0, 1], u2 in [0, 1)),
            scaled by 1/sqrt(K), then rounded to binary16
  scales    positive binary32, log-uniform over [2**lo, 2**hi): exponent
            lo + (draw >> 32) % (hi - lo), mantissa the low 23 bits of the draw
            (per-row / per-column quantization scales of the dequantizing
            epilogue)

Operand formats (the layout of the GEMM's operands):
  A   M x K, row-major, K contiguous        -> numpy array shape (M, K)
  B   K x N, column-major, K contiguous     -> returned as Bt, shape (N, K)
  int4 operands pack two signed 4-bit values per byte along K, the even k in
  the low nibble -> uint8 array shape (rows, K // 2)
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1
_CHUNK = 1 << 22

OPERAND_A = 1
OPERAND_B = 2


def config_seed(cfg_id: int, n: int, operand: int) -> int:
    """Seed of one operand of one workload: (cfg_id << 32) ^ (n << 8) ^ operand."""
    return ((cfg_id << 32) ^ (n << 8) ^ operand) & _M64


def splitmix64_scalar(seed: int, count: int) -> list[int]:
    """Plain Python big-int SplitMix64 stream (slow; used to check the vectorised one)."""
    out = []
    state = seed & _M64
    for _ in range(count):
        state = (state + GAMMA) & _M64
        z = state
        z = ((z ^ (z >> 30)) * MIX1) & _M64
        z = ((z ^ (z >> 27)) * MIX2) & _M64
        out.append(z ^ (z >> 31))
    return out


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Elements [start, start+count) of the SplitMix64 stream of `seed` as uint64."""
    out = np.empty(count, dtype=np.uint64)
    g = np.uint64(GAMMA)
    s = np.uint64(seed & _M64)
    m1 = np.uint64(MIX1)
    m2 = np.uint64(MIX2)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            hi = min(count, lo + _CHUNK)
            z = np.arange(start + lo + 1, start + hi + 1, dtype=np.uint64)
            z *= g
            z += s
            z ^= z >> np.uint64(30)
            z *= m1
            z ^= z >> np.uint64(27)
            z *= m2
            z ^= z >> np.uint64(31)
            out[lo:hi] = z
    return out


def _unit53(x: np.ndarray) -> np.ndarray:
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def int8_matrix(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols int8, uniform on [-128, 127]."""
    x = splitmix64(seed, rows * cols)
    return (x >> np.uint64(56)).astype(np.uint8).view(np.int8).reshape(rows, cols)


def int4_values(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols signed 4-bit values in [-8, 7], one per int8 element (unpacked)."""
    x = splitmix64(seed, rows * cols)
    return ((x >> np.uint64(60)).astype(np.int16) - 8).astype(np.int8).reshape(rows, cols)


def pack_int4(vals: np.ndarray) -> np.ndarray:
    """Pack signed 4-bit values along the last axis, two per byte, even index in the low nibble."""
    v = np.asarray(vals)
    if v.shape[-1] % 2:
        raise ValueError("int4 packing needs an even extent along K")
    if v.size and (v.min() < -8 or v.max() > 7):
        raise ValueError("int4 values must lie in [-8, 7]")
    u = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: uint8 (..., K/2) -> int8 (..., K)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def f16_uniform(rows: int, cols: int, seed: int) -> np.ndarray:
    """rows x cols binary16, U[-1, 1) drawn in fp64 and rounded to nearest even."""
    x = splitmix64(seed, rows * cols)
    return (2.0 * _unit53(x) - 1.0).astype(np.float16).reshape(rows, cols)


def f16_normal(rows: int, cols: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """rows x cols binary16, N(0, 1) * scale by Box-Muller, rounded to nearest even."""
    n = rows * cols
    out = np.empty(n, dtype=np.float16)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = splitmix64(seed, 2 * (hi - lo), start=2 * lo)
        u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = _unit53(x[1::2])
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
        out[lo:hi] = (z * scale).astype(np.float16)
    return out.reshape(rows, cols)


def f32_scales(n: int, seed: int, lo: int = -12, hi: int = -2) -> np.ndarray:
    """n positive binary32 scales, log-uniform over [2**lo, 2**hi)."""
    if not -126 <= lo < hi <= 128:
        raise ValueError("scale exponents must stay in the normal binary32 range")
    x = splitmix64(seed, n)
    e = (x >> np.uint64(32)) % np.uint64(hi - lo)
    bits = ((e.astype(np.int64) + lo + 127) << 23) | (x & np.uint64(0x7FFFFF)).astype(np.int64)
    return bits.astype(np.uint32).view(np.float32)


def operands(prec: str, m: int, n: int, k: int, seed_a: int, seed_b: int,
             dist: str = "uniform"):
    """A (M x K) and Bt (N x K) for one precision.

    prec: "f16" | "i8" | "i4".  For "i4" the arrays are packed (rows, K/2) uint8.
    dist (f16 only): "uniform" for U[-1,1], "normal" for N(0,1)/sqrt(K).
    """
    if prec == "f16":
        if dist == "normal":
            s = 1.0 / math.sqrt(k) if k else 1.0
            return f16_normal(m, k, seed_a, s), f16_normal(n, k, seed_b, s)
        return f16_uniform(m, k, seed_a), f16_uniform(n, k, seed_b)
    if prec == "i8":
        return int8_matrix(m, k, seed_a), int8_matrix(n, k, seed_b)
    if prec == "i4":
        return pack_int4(int4_values(m, k, seed_a)), pack_int4(int4_values(n, k, seed_b))
    raise ValueError(f"unknown precision {prec!r}")


def with_leading_dim(x: np.ndarray, ld: int, fill=0) -> np.ndarray:
    """Copy a (rows, cols) array into a (rows, ld) buffer, padding each row with `fill`."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    buf = np.full((rows, ld), fill, dtype=x.dtype)
    buf[:, :cols] = x
    return buf
