"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is the oracle's C source with one plausible error substituted
in (a transposed operand, a dropped term, a wrong sign, float accumulation,
a double rounding, ...). The copy is compiled on the host into a temporary
library and the pins of test_oracle.py are run against it; a mutant that
passes every pin would mean the pins cannot see that mistake.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build
import test_oracle as T

SRC = open(oracle_build.SRC).read()

MUTANTS = {
    "transposed_A": ("? A[(size_t)i * lda + k] : A[(size_t)k * lda + i]",
                     "? A[(size_t)k * lda + i] : A[(size_t)i * lda + k]"),
    "transB_ignored": ("? B[(size_t)k * ldb + j] : B[(size_t)j * ldb + k]",
                       "? B[(size_t)k * ldb + j] : B[(size_t)k * ldb + j]"),
    "dropped_last_k": ("for (int k = 0; k < K; ++k) {\n                const double a",
                       "for (int k = 0; k < K - 1; ++k) {\n                const double a"),
    "beta_sign": ("double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)crow[j];",
                  "double t = (beta == 0.0f) ? 0.0 : -(double)beta * (double)crow[j];"),
    "alpha_ignored": ("crow[j] = (float)((double)alpha * acc[j] + t);",
                      "crow[j] = (float)(acc[j] + t);"),
    "float_accumulation": ("acc[j] += a * (double)brow[j];",
                           "acc[j] = (float)(acc[j] + a * (double)brow[j]);"),
    "double_rounding": ("crow[j] = (float)((double)alpha * acc[j] + t);",
                        "crow[j] = (float)((double)alpha * (double)(float)acc[j] + t);"),
    "reads_c_when_beta_zero": ("double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)crow[j];",
                               "double t = (double)beta * (double)crow[j];"),
    "row_stride_uses_N": ("float *crow = &C[(size_t)i * ldc];", "float *crow = &C[(size_t)i * N];"),
    "k0_alpha_path_ignores_beta": ("*c = (beta == 0.0f) ? 0.0f : (float)((double)beta * (double)*c);",
                                   "*c = 0.0f;"),
}


def _pins():
    """The pin checks, each raising AssertionError on a wrong oracle."""
    yield "bruteforce", lambda: [T.bruteforce(ta, tb, trials=8) for ta, tb in T.OPS]
    yield "integer", lambda: T.test_integer_inputs_exact(
        T.W.C5A[3].with_(name="m", M=60, N=70, K=50, fill="int_rand", alpha=2.0, beta=-1.0))
    yield "identity", lambda: [T.test_identity(t) for t in "NT"]
    yield "permutation", T.test_permutation_rows_and_columns
    yield "ramp", T.test_ramp_closed_form
    yield "zeroA", T.test_zero_A_gives_beta_c
    yield "k0", T.test_k_zero_and_alpha_zero_scale_c
    yield "beta0", T.test_beta_zero_does_not_read_c
    yield "fp64", T.test_fp64_accumulation
    yield "one_rounding", T.test_single_final_rounding
    yield "transpose", T.test_transpose_of_product_bit_exact
    yield "copies", lambda: [T.test_explicit_transposed_copies(ta, tb) for ta, tb in T.OPS]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(old, new))
    lib_path = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, str(src), "-o", str(lib_path)], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._configure(ctypes.CDLL(str(lib_path))))
    failed = []
    for pin, fn in _pins():
        try:
            fn()
        except AssertionError:
            failed.append(pin)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    src = tmp_path / "same.c"
    src.write_text(SRC)
    lib_path = tmp_path / "libsame.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, str(src), "-o", str(lib_path)], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._configure(ctypes.CDLL(str(lib_path))))
    for _, fn in _pins():
        fn()
