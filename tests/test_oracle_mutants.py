"""Plant plausible mistakes in copies of the oracle source, on the CPU, and
check that the pins catch every one (no GPU).

Each mutant is a one-token edit of oracle/sdt_oracle.c built into a temporary
shared library; the real oracle is untouched.  A mutant that no pin rejects
would mean the pins leave that part of the oracle unchecked.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sdt_oracle.c")

MUTANTS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)\n        s += dec[a[k]]",
                          "for (int64_t k = 0; k + 1 < K; ++k)\n        s += dec[a[k]]"),
    "b_stride_ignored": ("B + n * ldb, K)", "B + n, K)"),
    "a_stride_is_k": ("A + m * lda, B", "A + m * K, B"),
    "squared_a": ("s += dec[a[k]] * dec[b[k]];", "s += dec[a[k]] * dec[a[k]];"),
    "fp32_accumulator": ("    double s = 0.0;\n    for (int64_t k = 0; k < K; ++k)\n        s += dec[a[k]]",
                         "    float s = 0.0f;\n    for (int64_t k = 0; k < K; ++k)\n        s += dec[a[k]]"),
    "sign_dropped": ("return sign ? -mag : mag;", "return mag;"),
    "subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "exponent_bias": ("expo - 25)", "expo - 24)"),
    "ties_away": ("(d == 0.5 && fmod(fl, 2.0) != 0.0)", "(d == 0.5)"),
    "ties_down": ("(d > 0.5 || (d == 0.5 && fmod(fl, 2.0) != 0.0))", "(d > 0.5)"),
    # (">" instead of ">=" would be an equivalent mutant: the rounding formula
    # itself carries the tie at 65520 up to the infinity encoding.)
    "overflow_threshold": ("a >= 65520.0", "a >= 65504.0"),
    "no_overflow_check": ("a >= 65520.0", "a >= INFINITY"),
    "subnormal_floor": ("if (E < -14)\n        E = -14;", "if (E < -15)\n        E = -15;"),
    "gemv_column_stride": ("const uint16_t* col = B + n * ldb;", "const uint16_t* col = B + n * K;"),
    "gemv_reads_x_twice": ("s += dec[x[k]] * dec[col[k]];", "s += dec[x[k]] * dec[x[k]];"),
    "gemv_kn_row_stride": ("dec[B[k * ldb + n]]", "dec[B[k * N + n]]"),
    "gemv_kn_transposed": ("dec[B[k * ldb + n]]", "dec[B[n * ldb + k]]"),
    "gemv_kn_first_row_dropped": ("for (int64_t k = 0; k < K; ++k)\n            s += dec[x[k]] * dec[B[k",
                                  "for (int64_t k = 1; k < K; ++k)\n            s += dec[x[k]] * dec[B[k"),
    "bf16_sign_dropped": ("return neg ? -v : v;", "return v;"),
    "bf16_subnormal_scale": ("ldexp((double)man, -133)", "ldexp((double)man, -134)"),
    "bf16_exponent_bias": ("ebits - 134)", "ebits - 133)"),
    "bf16_ties_away": ("(rem == 0.5 && fmod(lo, 2.0) == 1.0)", "(rem == 0.5)"),
    "bf16_ties_down": ("(rem > 0.5 || (rem == 0.5 && fmod(lo, 2.0) == 1.0))", "(rem > 0.5)"),
    "bf16_overflow_threshold": ("mag >= ldexp(255.5, 120)", "mag >= ldexp(255.0, 120)"),
    "bf16_subnormal_floor": ("if (P < -126)\n        P = -126;", "if (P < -127)\n        P = -127;"),
    "bf16_table_is_f16": ("return dtype == 1 ? g_dec_bf16 : (dtype == 0 ? g_dec : 0);",
                          "return dtype == 1 ? g_dec : (dtype == 0 ? g_dec : 0);"),
    "sample_swaps_index": ("dot_f64(dec, A + rows[i] * lda, B + cols[i] * ldb, K)",
                           "dot_f64(dec, A + rows[i] * lda, B + rows[i] * ldb, K)"),
}


def _build(name, src_text, tmp):
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib_{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-fopenmp", "-ffp-contract=off",
                    "-shared", "-o", so, c, "-lm"], check=True, capture_output=True)
    return so


@pytest.fixture(scope="module")
def tmpdir_mod():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    so = _build(name, src.replace(old, new), tmpdir_mod)
    o = oracle.Oracle(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, OverflowError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects mutant {name}"


def test_unmutated_copy_passes(tmpdir_mod):
    """Control: the same build recipe on the unmodified source passes every pin."""
    so = _build("control", open(SRC).read(), tmpdir_mod)
    o = oracle.Oracle(so)
    for pin in oracle_pins.ALL_PINS:
        pin(o)
