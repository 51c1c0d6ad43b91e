"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Each mutant is a one-line textual change to oracle/oracle.c (a dropped term,
a wrong sign, a transposed operand, a wrong exponent bias, float instead of
double, a skipped row ...).  The copy is compiled into a temporary directory
on the CPU; the real oracle is never modified.  A mutant that no pin catches
means the pins are too weak, and the test fails.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "drop_first_k": ("for (int64_t k = 0; k < jb->K; ++k) {\n                c += ai[k] * bj[k];",
                     "for (int64_t k = 1; k < jb->K; ++k) {\n                c += ai[k] * bj[k];"),
    "drop_last_k": ("for (int64_t k = 0; k < jb->K; ++k) {\n                c += ai[k] * bj[k];",
                    "for (int64_t k = 0; k + 1 < jb->K; ++k) {\n                c += ai[k] * bj[k];"),
    "wrong_sign": ("c += ai[k] * bj[k];", "c -= ai[k] * bj[k];"),
    "a_column_major": ("a[i * K + k] = elem(dtype, A, i * K + k);",
                       "a[i * K + k] = elem(dtype, A, k * M + i);"),
    "b_not_transposed": ("bt[j * K + k] = elem(dtype, B, k * N + j);",
                         "bt[j * K + k] = elem(dtype, B, j * K + k);"),
    "f16_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "f16_subnormal": ("v = ldexp((double)f, -24); ", "v = ldexp((double)f, -25); "),
    "f16_nan_as_inf": ("v = f ? NAN : INFINITY;\n    else\n        v = ldexp((double)(1024",
                       "v = INFINITY;\n    else\n        v = ldexp((double)(1024"),
    "bf16_subnormal": ("v = ldexp((double)f, -133);", "v = ldexp((double)f, -134);"),
    "bf16_exponent_field": ("int e = (b >> 7) & 0xff;", "int e = (b >> 8) & 0xff;"),
    "f32_bias": ("e - 150);", "e - 149);"),
    "s_signed": ("s += fabs(ai[k]) * fabs(bj[k]);", "s += ai[k] * fabs(bj[k]);"),
    "float_products": ("c += ai[k] * bj[k];", "c += (float)(ai[k] * bj[k]);"),
    "float_accumulator": ("double c = 0.0, s = 0.0;", "float c = 0.0f; double s = 0.0;"),
    "sampled_b_index": ("double b = elem(jb->dtype, jb->B, k * jb->N + j);",
                        "double b = elem(jb->dtype, jb->B, j * jb->K + k);"),
    "sampled_col_off_by_one": ("int64_t i = jb->rows[s], j = jb->cols[s];",
                               "int64_t i = jb->rows[s], j = (jb->cols[s] + 1) % jb->N;"),
    "i8_unsigned": ("return (double)((const int8_t *)p)[idx];",
                    "return (double)((const uint8_t *)p)[idx];"),
    "last_row_skipped": ("M * t / nthreads, M * (t + 1) / nthreads}",
                         "M * t / nthreads, M * (t + 1) / nthreads - (t == nthreads - 1)}"),
}


HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# Runs the pins against one compiled copy in a child process, so a mutant that
# crashes (an out-of-range index) is reported as caught instead of killing pytest.
CHILD = """
import sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, oracle_pins
lib = oracle.load({so!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:
        print("CAUGHT", pin.__name__, type(e).__name__)
        sys.exit(3)
print("ALL_PASS")
"""


def _build_copy(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found in oracle.c"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new, 1))
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(out=so, src=str(path))
    return so


def _run_pins(so):
    code = CHILD.format(root=ROOT, here=HERE, so=so)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600)


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    res = _run_pins(_build_copy(tmp_path, name, old, new))
    assert "ALL_PASS" not in res.stdout, f"no pin catches the '{name}' mutant"
    assert res.returncode != 0


def test_unmutated_copy_passes(tmp_path):
    # control: the same build path with no change passes every pin
    res = _run_pins(_build_copy(tmp_path, "none", "#include <math.h>", "#include <math.h>"))
    assert res.returncode == 0 and "ALL_PASS" in res.stdout, res.stdout + res.stderr
