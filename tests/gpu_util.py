"""Helpers for the GPU parity tests: padded device operands, guarded outputs,
whole-output and sampled-entry checks against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import oracle.matmul
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


def oracle_whole(prec, A, B, K, N=None, rowb=False):
    """The whole product from the oracle's matrix-product form (oracle/matmul.py):
    (R, S) for FP16, exact int64 for INT8 / INT4."""
    f = {"f16": oracle.matmul.gemm_f16, "i8": oracle.matmul.gemm_i8, "i4": oracle.matmul.gemm_i4}[prec]
    return f(A, B, K=K, N=N, rowb=rowb)


def check_whole(prec, A, B, K, C, what="", rowb=False):
    """Every element of C against the oracle: within 1e-3 * S for FP16, bit-exact
    for the integer paths."""
    ref = oracle_whole(prec, A, B, K, N=C.shape[1], rowb=rowb)
    if prec == "f16":
        assert_f16_close(C, ref[0], ref[1], what)
    else:
        assert_int_equal(C, ref, what)
    return ref


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
