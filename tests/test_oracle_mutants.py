"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins in test_oracle.py catch every one of them.

The mutants are built in a temporary directory on the CPU; the committed
oracle is never modified.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

MUTANTS = {
    "drop_last_k": ("for (k = 0; k < jb->K; ++k)", "for (k = 0; k < jb->K - 1; ++k)"),
    "nibble_order": ("(k & 1) ? (byte >> 4) : (byte & 0x0f)", "(k & 1) ? (byte & 0x0f) : (byte >> 4)"),
    "no_sign_extend": ("return v < 8 ? v : v - 16;", "return v;"),
    "subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "exponent_bias": ("ldexp((double)(1024 + frac), expo - 25)", "ldexp((double)(1024 + frac), expo - 24)"),
    "hidden_bit": ("(double)(1024 + frac)", "(double)(frac)"),
    "transposed_B_i8": ("    return rowmajor ? b[k * ldb + j] : b[j * ldb + k];",
                        "    return rowmajor ? b[k * ldb + j] : b[k * ldb + j];"),
    "B_uses_lda": ("b_i8(jb->B, jb->ldb, rm, k, j)", "b_i8(jb->B, jb->lda, rm, k, j)"),
    "i4_byte_stride": ("const uint8_t *a = (const uint8_t *)jb->A + i * (jb->lda / 2);",
                       "const uint8_t *a = (const uint8_t *)jb->A + i * jb->lda;"),
    "magnitude_signed": ("mag += fabs(prod);\n            }\n            r[j]", "mag += prod;\n            }\n            r[j]"),
    "subtract_product": ("acc += prod;\n                mag", "acc -= prod;\n                mag"),
    "f16_B_uses_lda": ("b_f16(jb->B, jb->ldb, rm, k, j)", "b_f16(jb->B, jb->lda, rm, k, j)"),
    "rowb_f16_as_colmajor": ("oracle_half_to_double(rowmajor ? b[k * ldb + j] : b[j * ldb + k])",
                             "oracle_half_to_double(rowmajor ? b[j * ldb + k] : b[j * ldb + k])"),
    "rowb_i4_packed_along_k": ("rowmajor ? s4_at(b + k * (ldb / 2), j)", "rowmajor ? s4_at(b + j * (ldb / 2), k)"),
    "rowb_i8_wrong_stride": ("    return rowmajor ? b[k * ldb + j] : b[j * ldb + k];",
                             "    return rowmajor ? b[k * (ldb - 1) + j] : b[j * ldb + k];"),
    "rowb_entries_colmajor": ("b_i8(B, ldb, 1, k, cols[t])", "b_i8(B, ldb, 0, k, cols[t])"),
    "dequant_swapped_scales": ("float c = dequant(S[i * lds + j], scale_a[i], scale_b[j]);",
                               "float c = dequant(S[i * lds + j], scale_a[j % M], scale_b[i % N]);"),
    "dequant_scale_product_first": ("    c = c * sa;\n    c = c * sb;", "    c = c * (sa * sb);"),
    "half_truncates": ("    if (rem > half || (rem == half && (q & 1u)))\n        q += 1u;", ""),
    "half_ties_away": ("(rem == half && (q & 1u))", "(rem == half)"),
    "half_no_binade_carry": ("        if (q == 0x800u) {\n            q = 0x400u;\n            he += 1;\n        }", ""),
    "entries_swap_rc": ("const int8_t *a = A + rows[t] * lda;\n        const int8_t *b = B + cols[t] * ldb;",
                        "const int8_t *a = A + cols[t] * lda;\n        const int8_t *b = B + rows[t] * ldb;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert old in source, f"mutation site for {name} no longer exists in the oracle"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                           str(src), "-lm", "-o", str(lib)])
    saved_lib, saved_path = oracle._lib, oracle.LIBRARY
    caught = []
    try:
        oracle._lib = None
        oracle.LIBRARY = str(lib)
        small = [(m, n, k) for m in (1, 3, 8) for n in (1, 2, 7) for k in (1, 4, 8)]
        for pin in pins.PINS:
            try:
                if pin is pins.pin_brute_force_tiny:
                    pin(small)
                else:
                    pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle._lib, oracle.LIBRARY = saved_lib, saved_path
    assert caught, f"no pin caught the planted mistake {name}"


# Planted mistakes in a copy of oracle/matmul.py, the whole-product form; each
# must make at least one of the MATMUL_PINS fail.
MATMUL_MUTANTS = {
    "nibble_order": ("nib[:, 0::2] = b & 0x0F\n    nib[:, 1::2] = b >> 4",
                     "nib[:, 0::2] = b >> 4\n    nib[:, 1::2] = b & 0x0F"),
    "no_sign_extend": ("nib = np.where(nib < 8, nib, nib - 16)", "nib = nib"),
    "magnitude_signed": ("return a @ b, np.abs(a) @ np.abs(b)", "return a @ b, np.abs(a @ b)"),
    "drop_last_k": ("        return x[:, :count]", "        return x[:, :max(count - 1, 0)]"),
    "rowb_read_as_colmajor": ("        b = decode(B, N)[:K]\n", "        b = decode(B, K)[:N].T\n"),
    "colmajor_read_as_rowb": ("        b = decode(B, K)[:N].T", "        b = decode(B, N)[:K]"),
    "negated_sum": ("    return np.rint(a @ b).astype(np.int64)", "    return np.rint(-(a @ b)).astype(np.int64)"),
}


@pytest.mark.parametrize("name", sorted(MATMUL_MUTANTS))
def test_matmul_mutant_is_caught(tmp_path, name):
    import importlib.util
    import oracle.matmul
    old, new = MATMUL_MUTANTS[name]
    text = open(oracle.matmul.__file__).read()
    assert old in text, f"mutation site for {name} no longer exists in oracle/matmul.py"
    path = tmp_path / f"matmul_{name}.py"
    path.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"matmul_mutant_{name}", path)
    mutant = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mutant)
    caught = []
    for pin in pins.MATMUL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            # a mutant that makes a pin's shapes inconsistent is caught too
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
