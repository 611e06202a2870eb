"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU), builds it into a
temporary library, swaps it in for the real one, and checks that at least one of the pin
tests in test_oracle.py / test_oracle_plan_fold.py now fails.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle as pins
import test_oracle_plan_fold as plan_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "value slice from the rope end": ("table[vrow[c]]", "table[vrow[c + 64]]"),
    "dropped k_scale on values": ("o[c] += w * (k_scale * table[vrow[c]]);",
                                  "o[c] += w * table[vrow[c]];"),
    "dropped softmax scale": ("score[j - a] = sm_scale * dot;", "score[j - a] = dot;"),
    "natural-log lse": ("lse[t] = (m + log(l)) / log(2.0);", "lse[t] = m + log(l);"),
    "max not subtracted in lse": ("lse[t] = (m + log(l)) / log(2.0);",
                                  "lse[t] = log(l) / log(2.0);"),
    "rope dims skipped in scores": ("for (int d = 0; d < ORACLE_KDIM; ++d)\n                dot",
                                    "for (int d = 0; d < ORACLE_VDIM; ++d)\n                dot"),
    "wrong page slot": ("j % ORACLE_PAGE) * ORACLE_KDIM;\n            double dot",
                        "(j + 1) % ORACLE_PAGE) * ORACLE_KDIM;\n            double dot"),
    "subnormal exponent": ("ldexp((double)mantissa / 8.0, -6)", "ldexp((double)mantissa / 8.0, -7)"),
    "exponent bias": ("exponent - 7);", "exponent - 8);"),
    "sign dropped": ("return sign ? -magnitude : magnitude;", "return magnitude;"),
    "merge weight base": ("double w = exp2(lse[s] - *lse_out);", "double w = exp(lse[s] - *lse_out);"),
    "plan cut not moved to the request start": ("cut[g] = voff[r];", "cut[g] = c;"),
    "plan cut not moved to the request end": ("cut[g] = end;", "cut[g] = c;"),
    "plan ignores min split": ("int64_t Gp = V / minp;", "int64_t Gp = V;"),
    "plan ignores max splits": ("if (Gp > max_splits)\n            Gp = max_splits;", ""),
    "plan cuts rounded up": ("int64_t c = g * V / Gp;", "int64_t c = (g * V + Gp - 1) / Gp;"),
    "plan group start off by one": ("if (start >= cut[g])", "if (start > cut[g])"),
    "plan heads not laid out": ("V += pages[r] > 0 ? a + pages[r] : 0;", "V += pages[r];"),
    "plan cut page counts the head": ("(int32_t)(cut[g] - voff[r] - a);", "(int32_t)(cut[g] - voff[r]);"),
    "plan item start skips the head": ("(work[2 * i + 1] > 0 ? a + work[2 * i + 1] : 0)",
                                       "work[2 * i + 1]"),
    "fixed groups rounded up": ("gstart[g] = (int32_t)(g * n / G);",
                                "gstart[g] = (int32_t)((g * n + G - 1) / G);"),
    "fixed remainder to the end": ("(int32_t)(s * q + (s < rem ? s : rem));", "(int32_t)(s * q);"),
    "item range ends a page early": ("work[2 * i + 3] : pages;", "work[2 * i + 3] : pages - 1;"),
}

PIN_TESTS = [
    pins.test_e4m3_table_matches_torch_all_codes,
    pins.test_e4m3_closed_values,
    pins.test_attend_matches_python_brute_force,
    lambda: pins.test_attend_matches_torch_float64_attention([1, 64, 65]),
    pins.test_uniform_keys_closed_form,
    pins.test_single_key,
    lambda: pins.test_split_merge_equals_no_split(0),
    pins.test_merge_two_equal_halves,
    plan_pins.test_plan_worked_example_two_requests,
    plan_pins.test_plan_worked_example_cuts_inside_a_request,
    plan_pins.test_plan_worked_example_moved_cuts,
    plan_pins.test_plan_worked_example_split_cost,
    plan_pins.test_plan_worked_example_row_tiles_and_max_splits,
    plan_pins.test_plan_fixed_mode,
    lambda: plan_pins.test_plan_properties_random(3),
    plan_pins.test_plan_exhaustive_small,
]


def build_mutant(tmp_path, old, new):
    src = open(SRC).read()
    assert old in src, old
    src = src.replace(old, new, 1)
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(src)
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", str(c), "-o",
                    str(so), "-lm"], check=True, capture_output=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    path = build_mutant(tmp_path, old, new)
    real = oracle._load()
    mutant = ctypes.CDLL(path)
    for fn in ("oracle_e4m3_value", "oracle_e4m3_table", "oracle_attend", "oracle_merge",
               "oracle_plan", "oracle_item_range"):
        f = getattr(mutant, fn)
        f.restype = getattr(real, fn).restype
        f.argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", mutant)
    failed = []
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError):
            failed.append(getattr(t, "__name__", "lambda"))
    assert failed, f"no pin caught the mutant: {name}"
