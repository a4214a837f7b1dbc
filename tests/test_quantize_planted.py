"""The offline oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle/quantize.py, plants one mistake by text
substitution (a rank off by one, a wrong comparison, a dropped weight, the
other tie, a missing rounding, a wrong index), loads the copy as a module
and runs the pins of test_quantize_pins.py against it.  At least one pin
must fail for every mutant; the unmodified oracle passes them all.
"""
import importlib.util
import os

import pytest

import test_quantize_pins as pins
from oracle import quantize as q_orig

SRC = q_orig.__file__

MUTANTS = {
    "tail_rank_off_by_one": ("n_tail = (n * tail_ppm) // 1_000_000", "n_tail = (n * tail_ppm) // 1_000_000 + 1"),
    "t_max_rank_off_by_one": ("t_max = int(flat[order[n - 1 - n_tail]])", "t_max = int(flat[order[n - n_tail - 2]])"),
    "outlier_test_inclusive": ("out = (v < lo) | (v > hi)\n    if sens", "out = (v <= lo) | (v >= hi)\n    if sens"),
    "negatives_not_reversed": ("return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000).astype(np.uint32)",
                               "return np.where(b & 0x8000, b & 0x7FFF, b | 0x8000).astype(np.uint32)"),
    "dense_keeps_outliers": ("dense = np.where(out, np.uint16(0), w).astype(np.uint16)", "dense = w.copy()"),
    "sensitive_rank_off_by_one": ("return flat[order[n - 1 - n_top]]", "return flat[order[n - n_top]]"),
    "sensitivity_ignored": ("out |= np.asarray(sens, dtype=np.float32) > np.float32(t_s)", "pass"),
    "dense_sensitivity_shifted": (
        "out[r, np.asarray(col[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)] = 0",
        "out[r, (np.asarray(col[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64) + 1) % out.shape[1]] = 0"),
    "unweighted_mean": ("c[j] = (wt[m] * x[m]).sum() / sw", "c[j] = x[m].mean()"),
    "start_misses_the_top": ("c = np.array([lo + j * (hi - lo) / (k - 1) for j in range(k)], dtype=np.float64)",
                             "c = np.array([lo + j * (hi - lo) / k for j in range(k)], dtype=np.float64)"),
    "ties_to_the_higher_centroid": ("return np.argmin(d, axis=1)  # argmin returns the first of equal minima",
                                    "return d.shape[1] - 1 - np.argmin(d[:, ::-1], axis=1)"),
    "codes_against_unrounded_centroids": ("codes[r] = nearest(x, f16_to_f64(lut[r])).astype(np.uint8)",
                                          "codes[r] = nearest(x, c).astype(np.uint8)"),
    "objective_without_weights": ("return (wt * (x - q) ** 2).sum(axis=1)", "return ((x - q) ** 2).sum(axis=1)"),
}


def _load(src_text: str, name: str):
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src_text, f"<{name}>", "exec"), mod.__dict__)
    return mod


def _battery():
    return [
        ("thresholds_known_order", pins.test_thresholds_of_a_known_order),
        ("signed_zero", pins.test_thresholds_signed_zero_order),
        ("extract", pins.test_extract_reconstructs_w),
        ("kmeans_start", pins.test_kmeans_keeps_data_that_equals_the_start),
        ("uniform_8", lambda: pins.test_kmeans_uniform_data_reaches_optimal_uniform_quantizer(8)),
        ("uniform_16", lambda: pins.test_kmeans_uniform_data_reaches_optimal_uniform_quantizer(16)),
        ("monotone", pins.test_kmeans_objective_never_increases),
        ("weighted", pins.test_weighted_centroid_moves_onto_dominant_value),
        ("beats_grid", pins.test_kmeans_beats_uniform_grid_on_heavy_tails),
        ("sens_threshold", pins.test_sensitive_threshold_of_a_known_order),
        ("union", pins.test_split_with_sensitive_values_is_the_union),
        ("zero_sensitivity", pins.test_zero_sensitivity_weights_take_no_part),
        ("ties", pins.test_kmeans_ties_go_to_the_lower_centroid),
        ("lut_rounding", pins.test_kmeans_codes_are_nearest_to_the_fp16_table),
        ("weighted_objective", pins.test_objective_weighs_each_error_by_its_sensitivity),
    ]


def _run_battery(mod, monkeypatch):
    monkeypatch.setattr(pins, "q", mod)
    failed = []
    for name, fn in _battery():
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmodified_oracle_passes_battery(monkeypatch):
    assert _run_battery(_load(open(SRC).read(), "quantize_copy"), monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site of {name} not found exactly once"
    mutant = _load(text.replace(old, new), f"quantize_{name}")
    failed = _run_battery(mutant, monkeypatch)
    assert failed, f"no pin caught the planted mistake {name}"
