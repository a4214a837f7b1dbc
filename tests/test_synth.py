"""Seeded input generator: determinism, row addressability and the stated
distributions (CPU only)."""
import numpy as np
import pytest

import synth


def test_determinism_and_stream_independence():
    k1 = synth.key(0, synth.stream_id(synth.KIND_CODES, 1, 0))
    k2 = synth.key(0, synth.stream_id(synth.KIND_CODES, 1, 1))
    a = synth.codes(k1, 64, 512, 3)
    assert np.array_equal(a, synth.codes(k1, 64, 512, 3))
    assert not np.array_equal(a, synth.codes(k2, 64, 512, 3))
    assert synth.key(1, 5) != synth.key(0, 5)


def test_codes_are_row_addressable_and_in_range():
    k = synth.key(3, 77)
    full = synth.codes(k, 40, 768, 4)
    for r in (0, 17, 39):
        assert np.array_equal(synth.codes(k, 1, 768, 4, row0=r)[0], full[r])
    assert full.max() < 16
    c3 = synth.codes(k, 40, 768, 3)
    assert c3.max() < 8


def test_codes_uniform():
    c = synth.codes(synth.key(0, 9), 256, 4096, 3)
    freq = np.bincount(c.ravel(), minlength=8) / c.size
    assert np.all(np.abs(freq - 0.125) < 0.002)


def test_generator_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-8, 5, 5000),
                        [65519.0, 65520.0, 2.0 ** -25, 3 * 2.0 ** -25]])
    ours = np.array([synth.f16_bits(t) for t in v], dtype=np.uint16)
    with np.errstate(over="ignore"):
        assert np.array_equal(ours, v.astype(np.float16).view(np.uint16))


def test_lut_sorted_normal():
    lut = synth.lut(synth.key(0, 11), 2000, 3)
    f = lut.view(np.float16).astype(np.float64)
    assert np.all(np.diff(f, axis=1) >= 0)
    assert abs(f.std() - 0.02) < 0.001 and abs(f.mean()) < 0.001
    unsorted = synth.lut(synth.key(0, 11), 2000, 3, sorted_=False)
    assert np.array_equal(np.sort(unsorted.view(np.float16), axis=1).view(np.uint16), lut)


def test_nnz_rounding():
    assert synth.nnz_bp(4096, 4096, 45) == 75497
    assert synth.nnz_bp(8192, 8192, 45) == 301990
    assert synth.nnz_bp(22016, 8192, 45) == 811598
    assert synth.nnz_bp(22016, 8192, 5) == 90178
    assert synth.nnz_bp(11008, 4096, 45) == 202899


def _check_csr(rp, col, rows, cols, nnz):
    assert rp[0] == 0 and rp[-1] == nnz and np.all(np.diff(rp) >= 0)
    for r in range(rows):
        c = col[rp[r]:rp[r + 1]].astype(np.int64)
        assert np.all(np.diff(c) > 0) and (c.size == 0 or c[-1] < cols)


def test_uniform_csr():
    rows, cols = 512, 2048
    nnz = synth.nnz_bp(rows, cols, 45)
    rp, col, val = synth.csr_uniform(synth.key(0, 1), synth.key(0, 2), rows, cols, nnz)
    _check_csr(rp, col, rows, cols, nnz)
    counts = np.diff(rp)
    assert abs(counts.mean() - 0.0045 * cols) < 0.1
    v = val.view(np.float16).astype(np.float64)
    assert abs(v.std() - 0.2) < 0.02


def test_uniform_csr_extremes():
    rp, col, _ = synth.csr_uniform(synth.key(0, 1), synth.key(0, 2), 8, 256, 8 * 256)
    _check_csr(rp, col, 8, 256, 8 * 256)
    assert np.all(np.diff(rp) == 256)
    rp, col, _ = synth.csr_uniform(synth.key(0, 1), synth.key(0, 2), 8, 256, 0)
    assert np.all(rp == 0) and col.size == 0


def test_zipf_csr_skew():
    rows, cols = 5120, 5120
    nnz = synth.nnz_bp(rows, cols, 45)
    rp, col, _ = synth.csr_zipf(synth.key(0, 3), synth.key(0, 4), synth.key(0, 5), rows, cols, nnz)
    _check_csr(rp, col, rows, cols, nnz)
    counts = np.diff(rp)
    assert counts.max() == cols           # a few rows fully dense (capped)
    assert 1 <= (counts == cols).sum() <= 10
    assert np.median(counts) <= 10        # most rows hold a handful
    assert np.percentile(counts, 99) >= 100


def test_workloads():
    assert [(m.rows, m.cols, m.bits) for m in synth.workload(1)] == [(4096, 4096, 3)]
    assert len(synth.workload(3)) == 7 and all(m.zipf for m in synth.workload(3))
    assert {m.batch for m in synth.workload(4, batch=8)} == {8}
    w5 = synth.workload(5, bits=4, density_bp=5)
    assert len(w5) == 560 and all(m.bits == 4 and m.density_bp == 5 for m in w5)
    total = sum(m.rows * m.cols for m in w5)
    assert total == 80 * (4 * 8192 * 8192 + 3 * 22016 * 8192)


def test_make_matrix_rows_regenerate():
    m = synth.make_matrix(synth.MatrixSpec("t", 130, 512, 4, batch=2), seed=0, workload=7, index=3)
    sel = [0, 64, 129]
    assert np.array_equal(synth.codes_rows(m, sel), m.codes[sel])
    assert m.x.shape == (2, 512) and m.lut.shape == (130, 16)
