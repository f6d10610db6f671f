"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a one-spot textual change to oracle/sgemm_oracle.c of the kind
a plausible slip would make (a dropped term, a wrong sign or index, a
transposed operand, a lost scale, an FP32 accumulator, a wrong field of a
16-bit format).  It is compiled on the
CPU into a temporary library and every pin runs against it; the test passes
only if some pin rejects the mutant.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins as pins

MUTANTS = {
    "drop_last_k_full": ("for (int k = 0; k < j->K; ++k) {\n      const double a",
                         "for (int k = 0; k < j->K - 1; ++k) {\n      const double a"),
    "drop_last_k_points": ("for (int k = 0; k < j->K; ++k) {\n      const double q",
                           "for (int k = 0; k < j->K - 1; ++k) {\n      const double q"),
    "beta_sign": ("v += j->beta * (double)j->C[(long)i * j->ldc + c];\n      r[c] = v;",
                  "v -= j->beta * (double)j->C[(long)i * j->ldc + c];\n      r[c] = v;"),
    "beta_sign_points": ("v += j->beta * (double)j->C[(long)i * j->ldc + c];\n    j->R[p] = v;",
                         "v -= j->beta * (double)j->C[(long)i * j->ldc + c];\n    j->R[p] = v;"),
    "reads_c_when_beta_zero": ("      if (j->beta != 0.0) v += j->beta * (double)j->C[(long)i * j->ldc + c];\n      r[c] = v;",
                               "      v += j->beta * (double)j->C[(long)i * j->ldc + c];\n      r[c] = v;"),
    "ldb_for_lda": ("j->A[(long)i * j->lda + k]", "j->A[(long)i * j->ldb + k]"),
    "b_index_transposed": (": j->B[(long)k * j->ldb + c]", ": j->B[(long)c * j->ldb + k]"),
    "ta_ignored": ("j->ta ? j->A[(long)k * j->lda + i]", "j->ta ? j->A[(long)i * j->lda + k]"),
    "tb_ignored": ("j->tb ? j->B[(long)c * j->ldb + k]", "j->tb ? j->B[(long)k * j->ldb + c]"),
    "flags_swapped": ("return (double)(j->ta ? j->A", "return (double)(j->tb ? j->A"),
    "points_drop_flags": ("  j.ta = ta != 0; j.tb = tb != 0;\n  j.R = r_out;", "  j.R = r_out;"),
    "alpha_dropped": ("double v = j->alpha * r[c];", "double v = r[c];"),
    "float_accumulator": ("r[c] += p;", "r[c] = (float)(r[c] + p);"),
    "float_product": ("const double p = a * b_at(j, k, c);",
                      "const double p = (float)(a * b_at(j, k, c));"),
    "t_signed": ("if (t) t[c] += fabs(p);", "if (t) t[c] += p;"),
    "row_offset": ("double *r = j->R + (long)i * j->ldr;",
                   "double *r = j->R + (long)(i > 0 ? i - 1 : 0) * j->ldr;"),
    # 16-bit formats
    "bf16_shift": ("(uint32_t)h << 16;", "(uint32_t)h << 15;"),
    "f16_bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "f16_no_hidden_bit": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)m, e - 25)"),
    "f16_subnormal_as_normal": ("v = ldexp((double)m, -24);",
                                "v = ldexp((double)(1024 + m), -25);"),
    "f16_sign_dropped": ("return s ? -v : v;", "return v;"),
    "f16_exponent_bits": ("e = (h >> 10) & 31", "e = (h >> 10) & 15"),
    "lowp_formats_swapped": ("return dt == DT_BF16 ? bf16_value(h)", "return dt == DT_F16 ? bf16_value(h)"),
    "lowp_ta_ignored": ("j->ta ? j->A16[(long)k * j->lda + i]", "j->ta ? j->A16[(long)i * j->lda + k]"),
    "lowp_tb_ignored": ("j->tb ? j->B16[(long)c * j->ldb + k]", "j->tb ? j->B16[(long)k * j->ldb + c]"),
    "lowp_b_ld": ("j->B16[(long)k * j->ldb + c]", "j->B16[(long)k * j->lda + c]"),
    # 8-bit formats
    "e4m3_sign_dropped": ("  return s != 0 ? -v : v;", "  return v;"),
    "e5m2_sign_dropped": ("  return (s != 0) ? -v : v;", "  return v;"),
    "e4m3_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    "e4m3_nan_rule": ("if (e == 15 && m == 7)", "if (e == 15)"),
    "e4m3_subnormal": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "e5m2_bias": ("ldexp((double)(4 + m), e - 17)", "ldexp((double)(4 + m), e - 16)"),
    "e5m2_fraction_bits": ("m = b & 3;", "m = b & 7;"),
    "fp8_formats_swapped": ("return dt == DT_E4M3 ? e4m3_value(b)", "return dt == DT_E5M2 ? e4m3_value(b)"),
    "fp8_ta_ignored": ("j->ta ? j->A8[(long)k * j->lda + i]", "j->ta ? j->A8[(long)i * j->lda + k]"),
    "fp8_b_index": ("j->B8[(long)k * j->ldb + c]", "j->B8[(long)c * j->ldb + k]"),
    "lowp_points_no_flags": ("  j.M = M; j.N = N; j.K = K;\n  j.ta = ta != 0; j.tb = tb != 0;\n  j.alpha = (double)alpha; j.beta = (double)beta;\n  j.dt = dt; j.A16 = A; j.B16 = B; j.C = C;\n  j.lda = lda; j.ldb = ldb; j.ldc = ldc;\n  j.npts",
                             "  j.M = M; j.N = N; j.K = K;\n  j.alpha = (double)alpha; j.beta = (double)beta;\n  j.dt = dt; j.A16 = A; j.B16 = B; j.C = C;\n  j.lda = lda; j.ldb = ldb; j.ldc = ldc;\n  j.npts"),
}


_RUNNER = r"""
import sys
sys.path.insert(0, sys.argv[1])
import oracle
from tests import oracle_pins as pins
lib = oracle.load(sys.argv[2])
caught = []
for pin in pins.ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError):
        caught.append(pin.__name__)
print("CAUGHT " + ",".join(caught))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SOURCE, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new), encoding="utf-8")
    lib_path = oracle.compile_library(str(path), str(tmp_path / f"lib{name}.so"))
    # A mutant may read out of bounds and crash: run the pins in a child process,
    # where a crash also counts as the mutant being caught.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-c", _RUNNER, root, lib_path],
                          capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        return  # crashed or raised: caught
    line = [l for l in proc.stdout.splitlines() if l.startswith("CAUGHT")][-1]
    caught = [c for c in line[len("CAUGHT "):].split(",") if c]
    assert caught, f"mutant {name} passed every pin"


# ---- the acceptance bound (oracle.error_bound) --------------------------------

BOUND_MUTANTS = {
    "unit_2^-23": ("2.0 ** -24", "2.0 ** -23"),
    "unit_2^-25": ("2.0 ** -24", "2.0 ** -25"),
    "k_squared": ("4.0 * max(int(K), 1) *", "4.0 * max(int(K), 1) * max(int(K), 1) *"),
    "k_sqrt": ("4.0 * max(int(K), 1) *", "4.0 * max(int(K), 1) ** 0.5 *"),
    "no_k_floor": ("4.0 * max(int(K), 1) *", "4.0 * int(K) *"),
    "factor_1": ("return 4.0 *", "return 1.0 *"),
    "factor_8": ("return 4.0 *", "return 8.0 *"),
    "beta_term_dropped": ("        scale = scale + np.abs(", "        scale = scale + 0 * np.abs("),
    "beta_term_always": ("    if beta != 0:\n        scale", "    if True:\n        scale"),
    "alpha_signed": ("scale = abs(float(alpha)) * t", "scale = float(alpha) * t"),
    "beta_signed": ("scale + np.abs(float(beta) * np.asarray(c_in, dtype=np.float64))",
                    "scale + float(beta) * np.asarray(c_in, dtype=np.float64)"),
}


def _bound_source():
    import inspect
    return inspect.getsource(oracle.error_bound)


@pytest.mark.parametrize("name", sorted(BOUND_MUTANTS))
def test_bound_mutant_is_caught(name):
    """A planted mistake in the acceptance bound fails at least one of the
    bound pins (tests/bound_pins.py)."""
    import numpy as np
    from tests import bound_pins
    src = _bound_source()
    old, new = BOUND_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    mutant = ns["error_bound"]
    caught = []
    for pin in bound_pins.ALL_BOUND_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, ZeroDivisionError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"bound mutant {name} passed every pin"


def test_bound_pins_pass_on_the_bound_itself():
    """The unmutated source, run the same way, passes every bound pin."""
    import numpy as np
    from tests import bound_pins
    ns = {"np": np}
    exec(_bound_source(), ns)
    for pin in bound_pins.ALL_BOUND_PINS:
        pin(ns["error_bound"])
