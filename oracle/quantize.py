"""CPU oracle for the offline steps upstream of the product: the
dense-and-sparse split of a weight matrix and the per-row (optionally
sensitivity-weighted) 1-D k-means that yields the codes and lookup tables.

TEST INFRASTRUCTURE: only the test suite and the benchmark's CPU-baseline
leg may import this module.  Plain numpy in fp64; it shares nothing with the
HIP path.

What it follows (SqueezeLLM: Dense-and-Sparse Quantization, summary page):
  - §3.4 "The Dense-and-Sparse Decomposition": W = D + S, S holds the
    weights below the T_min percentile or above the T_max percentile (e.g.
    0.2 and 99.8), D the rest with zeros where S has its entries; S in CSR.
    Its paragraph on extending the sparse matrix with sensitive values (and
    "Sparsity allocation" under the design choices): S also takes the
    weights of highest sensitivity (0.05%), whether or not they are
    outliers, so that the k-means of D is no longer pulled toward them.
  - §3.3, Eq. 1: non-uniform quantization as 1-D k-means of a row's values
    (k = 2^b centroids, each weight to its nearest centroid).
  - §3.3, Eq. 6 and "The weighted k-means algorithm in practice": per output
    channel (row); centroids start uniformly spaced over the value range (one
    of the two starts the page names; chosen here); each step assigns every
    weight to the nearest centroid by plain distance and moves each centroid
    to the sensitivity-weighted mean of its weights; the centroids are stored
    as fp16, each weight as the index of its centroid.

Readings (the pages leave these open):
  - The percentile of n values is the value of rank floor(n * p) in
    ascending order, p = tail_ppm / 1e6, ranks counted from 0 at each end
    (T_min = sorted[n_tail], T_max = sorted[n - 1 - n_tail]).  Values are
    ordered as IEEE binary16 bit patterns in total order (-0 before +0);
    a weight is an outlier when it compares below T_min or above T_max as a
    number.  Thresholds are per matrix.
  - Sensitive values: with n_top = floor(n * top_ppm / 1e6), T_s is the
    sensitivity of rank n - 1 - n_top in ascending total order, and a weight
    is sensitive when its sensitivity compares above T_s (n_top of them when
    the values are distinct).  S is the union of outliers and sensitive
    weights.  S's positions take no part in the clustering of D: their
    sensitivities are set to zero (dense_sensitivity), and a weight of zero
    sensitivity adds nothing to a centroid's weighted mean.  Their codes
    are still those nearest to D's value there, 0.
  - A fixed number of k-means steps; a centroid with no weights (or zero
    total sensitivity) stays where it is; ties in "nearest" go to the lower
    index.  After the steps the centroids are rounded to fp16 and every
    weight is assigned to the nearest fp16 centroid (the table the product
    reads), ties to the lower index.
"""
from __future__ import annotations

import numpy as np


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def total_order_key(bits: np.ndarray) -> np.ndarray:
    """Order-preserving unsigned key of binary16 bit patterns (IEEE total
    order: negatives reversed below +0)."""
    b = np.asarray(bits, dtype=np.uint32)
    return np.where(b & 0x8000, (~b) & 0xFFFF, b | 0x8000).astype(np.uint32)


def total_order_key32(bits: np.ndarray) -> np.ndarray:
    """Order-preserving unsigned key of binary32 bit patterns."""
    b = np.asarray(bits, dtype=np.uint32)
    return np.where(b & 0x80000000, ~b, b | 0x80000000).astype(np.uint32)


def thresholds(w_bits: np.ndarray, tail_ppm: int):
    """(T_min bits, T_max bits, number of outliers) of a matrix's fp16 values
    (§3.4 "The Dense-and-Sparse Decomposition": percentile thresholds)."""
    flat = np.asarray(w_bits, dtype=np.uint16).ravel()
    n = flat.size
    n_tail = (n * tail_ppm) // 1_000_000
    order = np.argsort(total_order_key(flat), kind="stable")
    t_min = int(flat[order[n_tail]])
    t_max = int(flat[order[n - 1 - n_tail]])
    v = f16_to_f64(flat)
    lo, hi = f16_to_f64(np.array([t_min]))[0], f16_to_f64(np.array([t_max]))[0]
    nnz = int(np.count_nonzero((v < lo) | (v > hi)))
    return t_min, t_max, nnz


def sensitive_threshold(sens: np.ndarray, top_ppm: int) -> np.float32:
    """T_s of an fp32 sensitivity matrix: the value of rank n - 1 - n_top in
    ascending total order, n_top = floor(n * top_ppm / 1e6)."""
    flat = np.asarray(sens, dtype=np.float32).ravel()
    n = flat.size
    n_top = (n * top_ppm) // 1_000_000
    order = np.argsort(total_order_key32(flat.view(np.uint32)), kind="stable")
    return flat[order[n - 1 - n_top]]


def sparse_mask(w_bits, t_min: int, t_max: int, sens=None, t_s=None) -> np.ndarray:
    """True where a weight goes to S: outside [T_min, T_max], or (given
    sensitivities) sensitivity above T_s."""
    v = f16_to_f64(w_bits)
    lo, hi = f16_to_f64(np.array([t_min]))[0], f16_to_f64(np.array([t_max]))[0]
    out = (v < lo) | (v > hi)
    if sens is not None:
        out |= np.asarray(sens, dtype=np.float32) > np.float32(t_s)
    return out


def split_thresholds(w_bits: np.ndarray, tail_ppm: int, sens: np.ndarray, top_ppm: int):
    """(T_min bits, T_max bits, T_s, nnz of S) with sensitive values."""
    t_min, t_max, _ = thresholds(w_bits, tail_ppm)
    t_s = sensitive_threshold(sens, top_ppm)
    nnz = int(np.count_nonzero(sparse_mask(w_bits, t_min, t_max, sens, t_s)))
    return t_min, t_max, t_s, nnz


def dense_sensitivity(sens: np.ndarray, row_ptr: np.ndarray, col: np.ndarray) -> np.ndarray:
    """The sensitivities with zeros at the entries of S (given as CSR)."""
    out = np.array(sens, dtype=np.float32, copy=True)
    for r in range(out.shape[0]):
        out[r, np.asarray(col[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)] = 0
    return out


def extract(w_bits: np.ndarray, t_min: int, t_max: int, sens=None, t_s=None):
    """W = D + S: CSR (row_ptr int32, col uint16, val fp16 bits; columns
    ascending within a row) of the weights outside [T_min, T_max] (and,
    given sensitivities, those above T_s), and D as fp16 bits with zeros
    where S has its entries."""
    w = np.asarray(w_bits, dtype=np.uint16)
    rows, cols = w.shape
    out = sparse_mask(w, t_min, t_max, sens, t_s)
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(out.sum(axis=1))
    r_idx, c_idx = np.nonzero(out)  # row-major, columns ascending
    col = c_idx.astype(np.uint16)
    val = w[r_idx, c_idx].astype(np.uint16)
    dense = np.where(out, np.uint16(0), w).astype(np.uint16)
    return row_ptr, col, val, dense


def kmeans_row(values: np.ndarray, weights: np.ndarray | None, k: int, iters: int):
    """Centroids (fp64, k) of one row after `iters` weighted Lloyd steps from
    uniformly spaced starts (§3.3, Eq. 1 / Eq. 6)."""
    x = np.asarray(values, dtype=np.float64)
    wt = np.ones_like(x) if weights is None else np.asarray(weights, dtype=np.float64)
    lo, hi = x.min(), x.max()
    c = np.array([lo + j * (hi - lo) / (k - 1) for j in range(k)], dtype=np.float64)
    for _ in range(iters):
        assign = nearest(x, c)
        for j in range(k):
            m = assign == j
            sw = wt[m].sum()
            if sw > 0:
                c[j] = (wt[m] * x[m]).sum() / sw
    return c


def nearest(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid for every value; ties to the lower index."""
    d = np.abs(np.asarray(x, dtype=np.float64)[:, None] - np.asarray(c, dtype=np.float64)[None, :])
    return np.argmin(d, axis=1)  # argmin returns the first of equal minima


def kmeans_lut(dense_bits: np.ndarray, sens: np.ndarray | None, bits: int, iters: int):
    """Per-row codes (uint8) and fp16 tables of D: k-means per row, centroids
    rounded to fp16, then every weight to its nearest fp16 centroid."""
    d = np.asarray(dense_bits, dtype=np.uint16)
    rows, cols = d.shape
    k = 1 << bits
    lut = np.empty((rows, k), dtype=np.uint16)
    codes = np.empty((rows, cols), dtype=np.uint8)
    for r in range(rows):
        x = f16_to_f64(d[r])
        c = kmeans_row(x, None if sens is None else sens[r], k, iters)
        lut[r] = f64_to_f16_bits(c)
        codes[r] = nearest(x, f16_to_f64(lut[r])).astype(np.uint8)
    return codes, lut


def objective(dense_bits, sens, codes, lut) -> np.ndarray:
    """Per-row weighted squared error sum_i F_i (w_i - LUT[code_i])^2 (Eq. 6;
    F = 1 without sensitivities)."""
    x = f16_to_f64(dense_bits)
    q = np.take_along_axis(f16_to_f64(lut), np.asarray(codes, dtype=np.int64), axis=1)
    wt = np.ones_like(x) if sens is None else np.asarray(sens, dtype=np.float64)
    return (wt * (x - q) ** 2).sum(axis=1)
