"""Planted mistakes in copies of the oracle must each be caught by a pin (CPU only).

Every mutant is the oracle's C source with one plausible slip (a dropped term,
a wrong sign or index, a transposed operand, a wrong tie rule ...), built into
a temporary library.  The test passes only if at least one pin from
``oracle_pins`` fails on that library.  The real oracle is never modified.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kmref.c")

MUTANTS = {
    "tie_to_highest": ("if (d < best) {", "if (d <= best) {"),
    "sign_of_difference": ("double diff = x[j] - c[j];", "double diff = x[j] + c[j];"),
    "dropped_square": ("d += diff * diff;", "d += fabs(diff);"),
    "centroid_stride": ("const double* c = C + k * D;", "const double* c = C + k;"),
    "transposed_points": ("x[j] = load_x(X, dtype, i * D + j);", "x[j] = load_x(X, dtype, j * N + i);"),
    "second_not_tracked": ("} else if (d < second) {", "} else if (0) {"),
    "mean_off_by_one": ("Cnew[k * D + j] = s[j] / (double)n;", "Cnew[k * D + j] = s[j] / (double)(n + 1);"),
    "empty_zeroed": ("if (Cnew != Cprev) memcpy(Cnew + k * D, Cprev + k * D, sizeof(double) * (size_t)D);",
                     "memset(Cnew + k * D, 0, sizeof(double) * (size_t)D);"),
    "sum_skips_first_column": ("for (int64_t j = 0; j < D; ++j) s[j] += load_x(X, dtype, i * D + j);",
                               "for (int64_t j = 1; j < D; ++j) s[j] += load_x(X, dtype, i * D + j);"),
    "round_truncates": ("double r = nearbyint(q);", "double r = trunc(q);"),
    "bf16_wrong_precision": ("case KMREF_X_BF16: out[i] = kmref_round(c, 8, -126, 127); break;",
                             "case KMREF_X_BF16: out[i] = kmref_round(c, 9, -126, 127); break;"),
    "f16_wrong_bias": ("v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    "objective_skips_last": ("for (int64_t i = 0; i < N; ++i) s += d1[i];",
                             "for (int64_t i = 0; i + 1 < N; ++i) s += d1[i];"),
    "no_fp32_state": ("for (size_t i = 0; i < kd; ++i) C[i] = kmref_round(C[i], 24, -126, 127);",
                      "for (size_t i = 0; i < kd; ++i) C[i] = kmref_round(C[i], 8, -126, 127);"),
    "counts_wrong_cluster": ("if (counts) counts[k] = n;", "if (counts) counts[k] = n + (k == 0);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut_src = tmp_path / "kmref_mut.c"
    mut_src.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libkmref_mut.so")
    oracle.build(out_path=lib_path, src_path=str(mut_src))
    O = oracle.Oracle(oracle.load(lib_path))
    caught = None
    for pin in oracle_pins.ALL_PINS:  # stop at the first pin that catches it
        try:
            pin(O)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught = pin.__name__
            break
    assert caught, f"no pin caught mutant {name}"
