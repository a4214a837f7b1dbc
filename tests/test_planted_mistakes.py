"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies the oracle's C source, plants one mistake by text
substitution (a dropped term, a wrong sign, a wrong index, a transposed
operand, a misplaced byte, a wrong rounding), compiles the copy into a
temporary directory and runs the pin tests against it.  At least one pin must
fail for every mutant; the unmodified oracle passes them all
(test_oracle_pins.py).
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sqllm_oracle.c")

MUTANTS = {
    "drop_sparse_term": (
        "acc += oracle_f16_to_f64(val[i]) * oracle_f16_to_f64(xb[col_idx[i]]);", "(void)0;"),
    "negated_sparse_term": (
        "acc += oracle_f16_to_f64(val[i]) * oracle_f16_to_f64(xb[col_idx[i]]);",
        "acc -= oracle_f16_to_f64(val[i]) * oracle_f16_to_f64(xb[col_idx[i]]);"),
    "dense_loop_drops_last_column": (
        "        if (with_dense)\n            for (int64_t c = 0; c < cols; ++c)",
        "        if (with_dense)\n            for (int64_t c = 0; c < cols - 1; ++c)"),
    "reversed_lut_index": (
        "acc += oracle_f16_to_f64(lut[r * k + code_row[c]])",
        "acc += oracle_f16_to_f64(lut[r * k + (k - 1 - code_row[c])])"),
    "transposed_activation": (
        "* oracle_f16_to_f64(xb[c]);", "* oracle_f16_to_f64(x[c * batch + b]);"),
    "sparse_column_off_by_one": (
        "oracle_f16_to_f64(xb[col_idx[i]]);", "oracle_f16_to_f64(xb[(col_idx[i] + 1) % cols]);"),
    "decoder_exponent_bias": (
        "else v = ldexp((double)(1024 + f), e - 25);", "else v = ldexp((double)(1024 + f), e - 24);"),
    "decoder_subnormal_scale": (
        "if (e == 0) v = ldexp((double)f, -24);", "if (e == 0) v = ldexp((double)f, -25);"),
    "encoder_ties_away_from_zero": (
        "if (rem > half || (rem == half && (kept & 1))) kept += 1;", "if (rem >= half) kept += 1;"),
    "row_contiguous_layout": (
        "return ((t * G + group) * P + q) * 1024 + l * 16 + m;",
        "return ((t * G + group) * 64 + l) * (16 * P) + q * 16 + m;"),
    "extra_pair_bits_reversed": (
        "v |= ((byte >> 6) & 3u) << (2 * k);", "v |= ((byte >> 6) & 3u) << (4 - 2 * k);"),
    "nibbles_swapped": (
        "codes[r * cols + c] = (uint8_t)((j % 2 ? v >> bits : v) & mask);",
        "codes[r * cols + c] = (uint8_t)((j % 2 ? v : v >> bits) & mask);"),
    "two_bit_pair_nibbles_swapped": (
        "return (packed[string_byte_offset(row, group, p / 2, cols, bits)] >> (4 * (p % 2))) & 0xFu;",
        "return (packed[string_byte_offset(row, group, p / 2, cols, bits)] >> (4 * (1 - p % 2))) & 0xFu;"),
    "extra_pairs_unit_stride": (
        "int64_t unit = p / 16, pu = p % 16, base = 12 * unit;",
        "int64_t unit = p / 16, pu = p % 16, base = 16 * unit;"),
    "normaliser_without_abs": (
        "sc += fabs(w[c]) * fabs(oracle_f16_to_f64(xb[c]));", "sc += w[c] * oracle_f16_to_f64(xb[c]);"),
}


def _battery():
    """(name, callable) for every pin, with fixed parameters."""
    b = [("f16_decoder", pins.test_f16_decoder_matches_numpy_on_all_patterns),
         ("f16_encoder", pins.test_f16_encoder_matches_numpy_round_to_nearest_even)]
    for case in pins._golden()["cases"]:
        b.append((case["name"], lambda c=case: pins.test_unpack_hand_derived_bytes(c)))
    for pat in pins._golden()["patterns"]:
        b.append((pat["name"], lambda p=pat: pins.test_unpack_hand_derived_patterns(p)))
    b.append(("roundtrip", lambda: pins.test_unpack_roundtrip_with_independent_packer(3, 65, 256)))
    for sparsity in ("5pct", "dense_row"):
        b.append((f"brute_{sparsity}", lambda s=sparsity: pins.test_product_matches_brute_force(3, 65, 512, 2, s)))
    b += [("constant_lut", pins.test_constant_lut_closed_form),
          ("affine_lut", pins.test_affine_lut_closed_form),
          ("single_code", pins.test_single_code_plus_sparse_closed_form),
          ("one_hot", pins.test_one_hot_activation_returns_a_weight_column),
          ("zero_lut", pins.test_zero_lut_is_plain_csr_spmv),
          ("integers", pins.test_integer_inputs_are_exact),
          ("normaliser", pins.test_normaliser_equals_result_for_nonnegative_inputs),
          ("spmv_add", pins.test_spmv_add_matches_scipy)]
    return b


def _run_battery():
    failed = []
    for name, fn in _battery():
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.fixture
def swap_oracle_library():
    saved = (oracle._lib, oracle._SO, oracle._F16_TABLE)

    def use(path):
        oracle._lib, oracle._SO, oracle._F16_TABLE = None, path, None

    yield use
    oracle._lib, oracle._SO, oracle._F16_TABLE = saved


def test_unmodified_oracle_passes_battery():
    assert _run_battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, swap_oracle_library):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-std=c99", "-shared", "-fPIC", "-o", so, str(path), "-lm"])
    swap_oracle_library(so)
    failed = _run_battery()
    assert failed, f"no pin caught the planted mistake {name}"
