"""The CPU oracle against its pins, and planted mistakes against the pins.

Runs without a GPU.  ``oracle_pins`` holds the pins; here every pin runs on
the oracle as built from ``oracle/gemv_oracle.c``, and then on copies of that
source with one plausible mistake planted in each, every one of which must
fail at least one pin.
"""

import json
import re
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def built_oracle():
    oracle.ensure_built()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(built_oracle, pin):
    pin(built_oracle)


# (name, pattern in gemv_oracle.c, replacement); each is a mistake a
# plausible implementation could make.
MUTANTS = [
    ("drop_last_term", r"k < K; \+\+k", "k < K - 1; ++k"),
    ("drop_first_term", r"int64_t k = 0; k < K", "int64_t k = 1; k < K"),
    ("wrong_sign", r"sum \+= a \* x;", "sum -= a * x;"),
    ("transposed_A", r"m \* lda \+ k", "k * lda + m"),
    ("lda_ignored", r"m \* lda \+ k", "m * K + k"),
    ("x_column_ignored", r"j \* ldx \+ k", "k"),
    ("x_stride_wrong", r"j \* ldx \+ k", "j * M + k"),
    ("bias_dropped", r"if \(bias != NULL\) sum \+= \(double\)bias\[m\];", ";"),
    ("bias_subtracted", r"sum \+= \(double\)bias\[m\]", "sum -= (double)bias[m]"),
    ("bias_wrong_index", r"bias\[m\]", "bias[0]"),
    ("output_row_major", r"Y\[j \* M \+ m\]", "Y[m * nvec + j]"),
    ("abs_not_taken", r"fabs\(a \* x\)", "(a * x)"),
    ("float_accumulator", r"double sum = 0\.0;", "float sum = 0.0f;"),
    ("f16_subnormal_scale", r"ldexp\(\(double\)frac, -24\)", "ldexp((double)frac, -25)"),
    ("f16_exponent_bias", r"expo - 25\)", "expo - 24)"),
    ("f16_hidden_bit", r"1024 \+ frac", "frac"),
    ("f16_sign_ignored", r"return sign \? -mag : mag;", "return mag;"),
    ("f16_nan_as_inf", r"frac == 0 \? INFINITY : NAN", "INFINITY"),
    ("bf16_shift", r"<< 16\)", "<< 15)"),
    ("f16_bf16_swapped", r"dtype == ORACLE_F16 \?", "dtype == ORACLE_BF16 ?"),
    ("f32_stride", r"4 \* i", "2 * i"),
    ("accepts_lda_below_K", r"lda < K \|\| ", ""),
    ("silu_wrong_sign", r"exp\(-g\)", "exp(g)"),
    ("silu_no_up", r"\)\) \* U\[m\];", "));"),
    ("silu_as_sigmoid", r"H\[m\] = g / ", "H[m] = 1.0 / "),
    ("gated_swapped", r"oracle_gemv\(dtype, Au,", "oracle_gemv(dtype, Ag,"),
    ("q8_unsigned", r"\(double\)b - 256\.0", "(double)b"),
    ("q8_scale_dropped", r"double y = s \* sum;", "double y = sum;"),
    ("q8_scale_first_row", r"\(double\)scale\[m\]", "(double)scale[0]"),
    ("q8_bias_scaled", r"double y = s \* sum;\n            if \(bias != NULL\) y \+= \(double\)bias\[m\];",
     "double y = sum;\n            if (bias != NULL) y += (double)bias[m];\n            y *= s;"),
    ("q8_abs_unscaled", r"fabs\(s\) \* abs_sum", "abs_sum"),
    ("q8_ldq_ignored", r"Q\[m \* ldq \+ k\]", "Q[m * K + k]"),
    ("q8_accepts_ldq_below_K", r"ldq < K \|\| ", ""),
]


@pytest.mark.parametrize("name,pattern,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, pattern, repl):
    src = oracle.SOURCE.read_text()
    mutated, n = re.subn(pattern, repl, src)
    assert n >= 1, f"mutation {name} no longer applies to the oracle source"
    c_file = tmp_path / "mutant.c"
    c_file.write_text(mutated)
    lib = oracle.build(source=c_file, output=tmp_path / f"lib_{name}.so")
    failed = _failing_pins_in_child(lib)
    assert failed, f"no pin catches the planted mistake {name}"


def _failing_pins_in_child(lib: Path) -> list[str]:
    """Run every pin on the library at ``lib`` in a child process: a mutant
    that reads out of bounds may crash, and a crash counts as caught."""
    here = Path(__file__).resolve().parent
    code = (
        "import json, sys; sys.path[:0] = [%r, %r];"
        "import oracle, oracle_pins;"
        "print(json.dumps(oracle_pins.failing_pins(oracle.Oracle(%r))))"
        % (str(here.parent), str(here), str(lib)))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True,
                          text=True, timeout=300)
    if proc.returncode != 0:
        return [f"crashed (exit {proc.returncode})"]
    return json.loads(proc.stdout.strip().splitlines()[-1])


def test_mutation_harness_passes_clean_copy(tmp_path):
    """The copy-and-compile path itself leaves a correct oracle correct."""
    c_file = tmp_path / "clean.c"
    shutil.copy(oracle.SOURCE, c_file)
    lib = oracle.build(source=c_file, output=tmp_path / "lib_clean.so")
    assert _failing_pins_in_child(lib) == []
