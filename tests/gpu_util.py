"""Helpers for the GPU parity tests: padded device operands, guarded outputs,
sampled-entry and Freivalds checks against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

F16_REL = 1e-3          # per-element bound |C - R| <= F16_REL * S
POISON = {"f16": np.float16(np.nan), "i8": np.int8(127), "i4": np.uint8(0x77)}
C_SENTINEL_BITS = 0x7FBADBAD  # a NaN pattern for fp32 C, an odd value for int32 C


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def ld_align(prec: str) -> int:
    """Leading-dimension multiple (in elements of the operand) the library requires."""
    return {"f16": 8, "i8": 16, "i4": 32}[prec]


def to_device_padded(torch, host: np.ndarray, ld_cols: int, fill, dev):
    """(rows, cols) host array -> device buffer (rows, ld_cols) padded with `fill`;
    returns the (rows, cols) view that is passed to the library."""
    rows, cols = host.shape
    buf = synth.with_leading_dim(host, ld_cols, fill)
    t = torch.from_numpy(buf).to(dev)
    return t[:, :cols]


def guarded_out(torch, M: int, N: int, ldc: int, dtype, dev, extra_rows: int = 3):
    """Output buffer (M + extra_rows, ldc) filled with the sentinel; returns (buf, view)."""
    buf = torch.empty((M + extra_rows, ldc), dtype=torch.int32, device=dev)
    buf.fill_(C_SENTINEL_BITS)
    buf = buf.view(dtype)
    return buf, buf[:M, :N]


def check_guard(torch, buf, M: int, N: int):
    bits = buf.view(torch.int32).cpu().numpy()
    outside = np.ones(bits.shape, dtype=bool)
    outside[:M, :N] = False
    bad = np.count_nonzero(bits[outside] != C_SENTINEL_BITS)
    assert bad == 0, f"{bad} stores outside the M x N block"


def assert_f16_close(C: np.ndarray, R: np.ndarray, S: np.ndarray, what: str = ""):
    C = C.astype(np.float64)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    err = np.abs(C - R)
    lim = F16_REL * S
    bad = err > lim
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {np.count_nonzero(bad)} elements beyond 1e-3*S, e.g. "
                             + ", ".join(f"{tuple(i)} got {C[tuple(i)]} want {R[tuple(i)]} S {S[tuple(i)]}"
                                         for i in idx))


def assert_int_equal(C: np.ndarray, ref: np.ndarray, what: str = ""):
    assert ref.min(initial=0) >= -(2 ** 31) and ref.max(initial=0) < 2 ** 31, f"{what}: oracle sum leaves int32"
    C = C.astype(np.int64)
    if not np.array_equal(C, ref):
        bad = np.argwhere(C != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {C[i]} want {ref[i]}")


def oracle_full(prec, A, Bt, K):
    if prec == "f16":
        return oracle.gemm_f16(A, Bt, K=K)
    if prec == "i8":
        return oracle.gemm_i8(A, Bt, K=K)
    return oracle.gemm_i4(A, Bt, K=K)


def sample_positions(M: int, N: int, count: int, seed: int, tiles=(256, 128, 64, 32)):
    """Random positions plus every tile-edge row/column pair and the corners."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, count))
    cols = list(rng.integers(0, N, count))
    edge_r = sorted({x for t in tiles for b in range(0, M, t) for x in (b, min(b + t - 1, M - 1))} | {M - 1})
    edge_c = sorted({x for t in tiles for b in range(0, N, t) for x in (b, min(b + t - 1, N - 1))} | {N - 1})
    er = rng.choice(edge_r, size=min(len(edge_r), 256), replace=False)
    ec = rng.choice(edge_c, size=min(len(edge_c), 256), replace=False)
    for r in er:
        rows.append(int(r))
        cols.append(int(rng.integers(0, N)))
    for c in ec:
        rows.append(int(rng.integers(0, M)))
        cols.append(int(c))
    for r in (0, M - 1):
        for c in (0, N - 1):
            rows.append(r)
            cols.append(c)
    return np.array(rows, np.int64), np.array(cols, np.int64)


def check_sampled(prec, A, Bt, K, C, rows, cols, what=""):
    got = C[rows, cols]
    if prec == "f16":
        R, S = oracle.entries_f16(A, Bt, rows, cols, K=K)
        assert_f16_close(got, R, S, what)
    elif prec == "i8":
        assert_int_equal(got, oracle.entries_i8(A, Bt, rows, cols, K=K), what)
    else:
        assert_int_equal(got, oracle.entries_i4(A, Bt, rows, cols, K=K), what)


def freivalds_int(prec, A, Bt, K, C, seed, rounds=2):
    """Exact integer check C x == A (B x) over the whole matrix (int64, no overflow for
    |x| <= 2^20 at the sizes used here)."""
    if prec == "i4":
        Av = synth.unpack_int4(A)[:, :K].astype(np.int64)
        Bv = synth.unpack_int4(Bt)[:, :K].astype(np.int64)
    else:
        Av = A[:, :K].astype(np.int64)
        Bv = Bt[:, :K].astype(np.int64)
    C64 = C.astype(np.int64)
    rng = np.random.default_rng(seed)
    for _ in range(rounds):
        x = rng.integers(-(2 ** 20), 2 ** 20, C.shape[1], dtype=np.int64)
        lhs = C64 @ x
        rhs = Av @ (Bv.T @ x)
        assert np.array_equal(lhs, rhs), f"Freivalds check failed ({prec})"


def freivalds_f16(A, Bt, K, C, seed, rounds=2):
    """Necessary condition of the per-element bound over the whole matrix:
    for x in {-1, +1}^N, |C x - A (B x)| <= 1e-3 * |A| (|B| 1) + fp64 slack."""
    Ad = A[:, :K].astype(np.float64)
    Bd = Bt[:, :K].astype(np.float64)
    Cd = C.astype(np.float64)
    N = C.shape[1]
    sum_s = np.abs(Ad) @ (np.abs(Bd).T @ np.ones(N))
    bound = F16_REL * sum_s
    # fp64 rounding of the three products: below (2N + K) unit roundoffs of sum_s
    slack = (2 * N + K + 4) * 2.0 ** -52 * sum_s
    rng = np.random.default_rng(seed)
    for _ in range(rounds):
        x = rng.choice([-1.0, 1.0], size=N)
        diff = np.abs(Cd @ x - Ad @ (Bd.T @ x))
        assert np.all(diff <= bound + slack), f"f16 row-sum bound violated, worst excess {np.max(diff - bound)}"
