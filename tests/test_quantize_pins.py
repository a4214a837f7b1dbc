"""Pins of the offline oracle (oracle/quantize.py) against facts fixed by the
pages and by the mathematics, not by retyping its code (CPU only).

  - thresholds of a matrix whose sorted order is known by construction;
  - W = D + S exactly, CSR in row order, D zero where S has entries;
  - k-means: data equal to the starting centroids stays put with zero error;
    uniform data converges to the optimal uniform quantizer's centres
    (2j+1)/(2k); the objective never increases from step to step; a
    centroid's cluster dominated by one heavily weighted value moves onto it
    (Eq. 6); the k-means table beats a uniform grid on heavy-tailed rows.
"""
import numpy as np
import pytest

from oracle import quantize as q
from seeds import stable_seed


def f16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_thresholds_of_a_known_order():
    rng = np.random.default_rng(stable_seed("thr"))
    vals = np.unique(rng.normal(0, 1, 5000).astype(np.float16))  # distinct fp16 values, ascending
    n = vals.size
    mat = rng.permutation(vals).view(np.uint16).reshape(1, n)
    for ppm in (2000, 50000, 0):
        t_min, t_max, nnz = q.thresholds(mat, ppm)
        n_tail = n * ppm // 1_000_000
        assert t_min == int(vals.view(np.uint16)[n_tail])
        assert t_max == int(vals.view(np.uint16)[n - 1 - n_tail])
        assert nnz == 2 * n_tail  # distinct values: exactly n_tail below and above


def test_thresholds_signed_zero_order():
    # -0 sorts before +0; both compare equal as numbers, so neither is an outlier
    mat = np.array([[0x8000, 0x0000, 0x3C00, 0xBC00]], dtype=np.uint16)  # -0, +0, 1, -1
    t_min, t_max, nnz = q.thresholds(mat, 250000)  # one value per tail
    assert (t_min, t_max) == (0x8000, 0x0000)
    assert nnz == 2  # -1 and 1


def test_extract_reconstructs_w():
    rng = np.random.default_rng(stable_seed("extract"))
    w = f16(rng.standard_t(3, (37, 300)) * 0.02).reshape(37, 300)
    t_min, t_max, nnz = q.thresholds(w, 20000)
    rp, col, val, dense = q.extract(w, t_min, t_max)
    assert rp[0] == 0 and rp[-1] == nnz == col.size == val.size
    assert np.all(np.diff(rp) >= 0)
    s = np.zeros(w.shape, dtype=np.float64)
    for r in range(w.shape[0]):
        cs = col[rp[r]:rp[r + 1]].astype(np.int64)
        assert np.all(np.diff(cs) > 0)
        s[r, cs] = q.f16_to_f64(val[rp[r]:rp[r + 1]])
    d = q.f16_to_f64(dense)
    assert np.array_equal(d + s, q.f16_to_f64(w))
    assert np.all(d[s != 0] == 0)
    lo, hi = q.f16_to_f64(np.array([t_min, t_max]))
    assert np.all((d >= lo) & (d <= hi) | (d == 0))


def test_kmeans_keeps_data_that_equals_the_start():
    x = np.repeat(np.arange(8, dtype=np.float64), 5)
    c = q.kmeans_row(x, None, 8, 10)
    assert np.array_equal(c, np.arange(8, dtype=np.float64))
    codes, lut = q.kmeans_lut(f16(x).reshape(1, -1), None, 3, 10)
    assert np.all(q.objective(f16(x).reshape(1, -1), None, codes, lut) == 0)


@pytest.mark.parametrize("k", [8, 16])
def test_kmeans_uniform_data_reaches_optimal_uniform_quantizer(k):
    x = (np.arange(20000) + 0.5) / 20000  # uniform on [0, 1]
    c = q.kmeans_row(x, None, k, 400)
    assert np.allclose(c, (2 * np.arange(k) + 1) / (2 * k), atol=2e-3)


def test_kmeans_objective_never_increases():
    rng = np.random.default_rng(stable_seed("mono"))
    x = rng.standard_t(4, 3000) * 0.02
    wt = rng.exponential(1.0, 3000)
    prev = np.inf
    for it in range(12):
        c = q.kmeans_row(x, wt, 8, it)
        obj = (wt * (x - c[q.nearest(x, c)]) ** 2).sum()
        assert obj <= prev * (1 + 1e-12)
        prev = obj


def test_weighted_centroid_moves_onto_dominant_value():
    x = np.array([0.0, 0.1, 0.2, 10.0, 10.5, 11.0])
    wt = np.array([1.0, 1e9, 1.0, 1.0, 1.0, 1.0])
    c = q.kmeans_row(x, wt, 2, 20)
    assert abs(c[0] - 0.1) < 1e-6
    assert abs(c[1] - 10.5) < 1e-12


def test_kmeans_beats_uniform_grid_on_heavy_tails():
    rng = np.random.default_rng(stable_seed("rtn"))
    w = f16(rng.standard_t(3, (8, 2048)) * 0.02).reshape(8, 2048)
    codes, lut = q.kmeans_lut(w, None, 3, 20)
    err_km = q.objective(w, None, codes, lut)
    x = q.f16_to_f64(w)
    for r in range(8):
        grid = np.linspace(x[r].min(), x[r].max(), 8)
        err_u = ((x[r] - grid[q.nearest(x[r], grid)]) ** 2).sum()
        assert err_km[r] < err_u


def test_sensitive_threshold_of_a_known_order():
    rng = np.random.default_rng(stable_seed("sens-thr"))
    vals = np.unique(rng.exponential(1.0, 4000).astype(np.float32))  # distinct, ascending
    n = vals.size
    mat = rng.permutation(vals).reshape(4, n // 4) if n % 4 == 0 else rng.permutation(vals).reshape(1, n)
    for ppm in (500, 50000, 0):
        t_s = q.sensitive_threshold(mat, ppm)
        n_top = n * ppm // 1_000_000
        assert t_s == vals[n - 1 - n_top]
        assert np.count_nonzero(mat > t_s) == n_top


def test_split_with_sensitive_values_is_the_union():
    """Planted outliers O (5 on each tail) and planted most-sensitive weights
    P (3, one of them also an outlier): S is exactly O | P."""
    rng = np.random.default_rng(stable_seed("union"))
    rows, cols = 20, 100
    w = rng.uniform(-0.01, 0.01, (rows, cols))
    flat = rng.permutation(rows * cols)
    o_pos, p_pos = flat[:10], np.concatenate([flat[:1], flat[10:12]])
    w.ravel()[o_pos[:5]] = [1.0, 1.5, 2.0, 2.5, 3.0]
    w.ravel()[o_pos[5:]] = [-1.0, -1.5, -2.0, -2.5, -3.0]
    w_bits = f16(w).reshape(rows, cols)
    sens = rng.uniform(0, 1, (rows, cols)).astype(np.float32)
    sens.ravel()[p_pos] = [10.0, 11.0, 12.0]
    t_min, t_max, t_s, nnz = q.split_thresholds(w_bits, 2500, sens, 1500)   # 5 per tail, top 3
    want = set(o_pos.tolist()) | set(p_pos.tolist())
    assert nnz == len(want) == 12
    rp, col, val, dense = q.extract(w_bits, t_min, t_max, sens, t_s)
    got = {int(r) * cols + int(c) for r in range(rows) for c in col[rp[r]:rp[r + 1]]}
    assert got == want
    s = np.zeros((rows, cols))
    for r in range(rows):
        s[r, col[rp[r]:rp[r + 1]].astype(np.int64)] = q.f16_to_f64(val[rp[r]:rp[r + 1]])
    assert np.array_equal(q.f16_to_f64(dense) + s, q.f16_to_f64(w_bits))
    ds = q.dense_sensitivity(sens, rp, col)
    mask = np.zeros(rows * cols, bool)
    mask[list(want)] = True
    mask = mask.reshape(rows, cols)
    assert np.all(ds[mask] == 0) and np.array_equal(ds[~mask], sens[~mask])


def test_zero_sensitivity_weights_take_no_part():
    """A weight of zero sensitivity moves no centroid: the same centroids as
    clustering without it (its value inside the row's range)."""
    rng = np.random.default_rng(stable_seed("zero-sens"))
    x = rng.normal(0, 1, 3000)
    wt = rng.exponential(1.0, 3000)
    inner = np.flatnonzero((x > np.sort(x)[10]) & (x < np.sort(x)[-10]))[:200]
    wt[inner] = 0
    keep = wt > 0
    c_all = q.kmeans_row(x, wt, 8, 15)
    c_sub = q.kmeans_row(x[keep], wt[keep], 8, 15)
    assert np.allclose(c_all, c_sub, rtol=1e-12, atol=0)


def test_kmeans_ties_go_to_the_lower_centroid():
    """A weight halfway between two centroids takes the lower one, in the
    assignment steps and in the final codes.  Row 0, 0.5, 3 at 2 bits with no
    steps: the centroids stay at the uniform start 0, 1, 2, 3."""
    assert int(q.nearest(np.array([0.5]), np.array([0.0, 1.0]))[0]) == 0
    row = f16([0.0, 0.5, 3.0]).reshape(1, 3)
    codes, lut = q.kmeans_lut(row, None, 2, 0)
    assert np.array_equal(q.f16_to_f64(lut[0]), [0.0, 1.0, 2.0, 3.0])
    assert codes[0].tolist() == [0, 0, 3]


def test_kmeans_codes_are_nearest_to_the_fp16_table():
    """Codes follow the stored fp16 table, not the fp64 centroids.  Row 0,
    1001.5, 6008 at 2 bits with no steps: centroid 1 is 6008/3 = 2002.67,
    stored as 2003, so 1001.5 sits exactly halfway between 0 and 2003 (tie:
    code 0), while against 2002.67 it would be nearer code 1."""
    row = f16([0.0, 1001.5, 6008.0]).reshape(1, 3)
    codes, lut = q.kmeans_lut(row, None, 2, 0)
    assert q.f16_to_f64(lut[0])[1] == 2003.0
    assert codes[0].tolist() == [0, 0, 3]


def test_objective_weighs_each_error_by_its_sensitivity():
    """Eq. 6: sum of F_i (w_i - Q(w_i))^2, by hand: weights 1 and 2 both coded
    to centroid 0 with sensitivities 3 and 5 -> 3*1 + 5*4 = 23."""
    d = f16([1.0, 2.0]).reshape(1, 2)
    lut = f16([0.0, 10.0, 20.0, 30.0]).reshape(1, 4)
    codes = np.zeros((1, 2), np.uint8)
    assert q.objective(d, np.array([[3.0, 5.0]]), codes, lut)[0] == 23.0
    assert q.objective(d, None, codes, lut)[0] == 5.0
