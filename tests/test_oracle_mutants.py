"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a private copy of oracle/oracle.c (a
dropped term, a wrong sign, a transposed operand, a wrong leading dimension,
an off-by-one exponent bias, ties rounded away from even, ...), compiles it
with gcc into a temporary library, swaps it in for the real one and runs the
pin tests of test_oracle_formats.py / test_oracle_gemm.py against it.  Every
mutant must fail at least one pin.  All of this runs on the CPU.
"""
import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_formats as tf
from tests import test_oracle_gemm as tg

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("dropped_first_term", "for (int64_t k = 0; k < K; ++k) {\n      const double a = arow[k];",
     "for (int64_t k = 1; k < K; ++k) {\n      const double a = arow[k];"),
    ("wrong_sign", "c[j] += p;", "c[j] -= p;"),
    ("transposed_B", "const double p = a * b[j]; /* exact product */",
     "const double p = a * Bd[(j * K + k) % (K * N)]; (void)b;"),
    ("wrong_lda", "load_bits(A, i * K + k, f.bytes)",
     "load_bits(A, (i * N + k) % (M * K), f.bytes)"),
    ("normal_bias_off_by_one", "(int)e - f->bias - f->man_bits)",
     "(int)e - f->bias - f->man_bits + 1)"),
    ("subnormal_exponent", "ldexp((double)m, 1 - f->bias - f->man_bits)",
     "ldexp((double)m, -f->bias - f->man_bits)"),
    ("ties_away", "(frac == 0.5 && fmod(r, 2.0) != 0.0)", "(frac == 0.5)"),
    ("abs_bound_signed", "ca[j] += fabs(p);", "ca[j] += p;"),
    ("scale_ignored", "for (int64_t j = 0; j < N; ++j) c[j] *= scale;", ""),
    ("e4m3_as_ieee", "case ORC_E4M3: *f = (orc_fmt){4, 3, 7, 0, 1};",
     "case ORC_E4M3: *f = (orc_fmt){4, 3, 7, 1, 1};"),
    ("bf16_bias", "case ORC_BF16: *f = (orc_fmt){8, 7, 127, 1, 2};",
     "case ORC_BF16: *f = (orc_fmt){8, 7, 126, 1, 2};"),
    ("accumulator_not_cleared", "for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; ca[j] = 0.0; }",
     "for (int64_t j = 0; j < N; ++j) { c[j] = (i == 0) ? 1.0 : 0.0; ca[j] = 0.0; }"),
    ("last_term_dropped_in_elems", "for (int64_t k = 0; k < K; ++k) {\n      const double p = decode_bits",
     "for (int64_t k = 0; k + 1 < K; ++k) {\n      const double p = decode_bits"),
    ("i64_twin_transposed", "(int64_t)B[k * N + j]", "(int64_t)B[(j * K + k) % (K * N)]"),
]

PINS = [
    (tf.test_decode_f16_exhaustive, ()),
    (tf.test_decode_bf16_exhaustive, ()),
    (tf.test_decode_fp8_format_landmarks, ()),
    (tf.test_worked_example_encoding_table, ()),
    (tf.test_worked_example_2048_plus_1, ()),
    (tf.test_round_ties_to_even_f16, ()),
    (tg.test_i64_twin_hand_example, ()),
    (tg.test_identity, ("f16",)),
    (tg.test_all_ones_gives_K, ("f16", 256)),
    (tg.test_unit_selector_picks_row_of_B, ()),
    (tg.test_integer_inputs_match_int64_twin, ("f16", (37, 29, 53))),
    (tg.test_integer_inputs_match_int64_twin, ("e4m3", (37, 29, 53))),
    (tg.test_grid_inputs_exact, ("bf16",)),
    (tg.test_random_vs_numpy_fp64, ("f16",)),
    (tg.test_scale_is_applied, ()),
    (tg.test_rows_and_elems_agree_with_full, ()),
]


@contextlib.contextmanager
def _swapped(lib):
    saved = oracle._lib
    oracle._lib = lib
    try:
        yield
    finally:
        oracle._lib = saved


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", "-w", "-o", str(so), str(path), "-lm"], check=True)
    return oracle.bind(ctypes.CDLL(str(so)))


def test_unmutated_oracle_passes_the_pins():
    for fn, args in PINS:
        fn(*args)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build_mutant(tmp_path, name, old, new)
    caught = []
    with _swapped(lib):
        for fn, args in PINS:
            try:
                fn(*args)
            except (AssertionError, ValueError):
                caught.append(fn.__name__)
                break
    assert caught, f"no pin failed for the planted mistake {name!r}"
