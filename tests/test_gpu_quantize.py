"""Parity of the offline dense-and-sparse split and the per-row k-means
(through the C ABI) with oracle/quantize.py.

Bit-exact everywhere: the thresholds, the outlier count, the CSR arrays and
D are integer work decided by fp16 comparisons, which both sides make
exactly; the k-means tables and codes are fp64 arithmetic on both sides, so
they differ only if a weight lies within rounding of a midpoint between two
centroids (none does in these inputs).  At full layer size the thresholds
are checked by their rank property and the k-means on sampled rows.
Inputs: heavy-tailed (Student-t, 4 degrees of freedom) fp16 weights at the
scale of LLaMA linear layers, seeded.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import quantize as q
from seeds import stable_seed
from gpu_util import assert_close, dev_to_u16, nw, step, u16_to_dev

pytestmark = pytest.mark.gpu


def heavy(tag, rows, cols, df=4, scale=0.02):
    rng = np.random.default_rng(stable_seed(tag))
    return (rng.standard_t(df, (rows, cols)) * scale).astype(np.float16).view(np.uint16)


def split_on_gpu(w, ppm):
    wd = u16_to_dev(w)
    t_min, t_max, t_s, nnz = nw().outlier_thresholds(wd, ppm)
    assert t_s == float("inf")
    rp, col, val, dense = nw().outlier_extract(wd, t_min, t_max, nnz)
    torch.cuda.synchronize()
    return (t_min, t_max, nnz, rp.cpu().numpy(), dev_to_u16(col) if nnz else np.zeros(0, np.uint16),
            dev_to_u16(val) if nnz else np.zeros(0, np.uint16), dev_to_u16(dense))


def split_sens_on_gpu(w, sens, ppm, top_ppm):
    """(t_min, t_max, t_s, nnz), (row_ptr, col, val, dense, sens_dense) as numpy."""
    wd, sd = u16_to_dev(w), torch.from_numpy(sens).cuda()
    t_min, t_max, t_s, nnz = nw().outlier_thresholds(wd, ppm, sd, top_ppm)
    rp, col, val, dense, sdense = nw().outlier_extract(wd, t_min, t_max, nnz, sd, t_s)
    torch.cuda.synchronize()
    arrays = (rp.cpu().numpy(), dev_to_u16(col) if nnz else np.zeros(0, np.uint16),
              dev_to_u16(val) if nnz else np.zeros(0, np.uint16), dev_to_u16(dense), sdense.cpu().numpy())
    return (t_min, t_max, np.float32(t_s), nnz), arrays


def fisher_like(tag, rows, cols):
    """Non-negative, heavy-tailed sensitivities (squared normal times a
    log-normal per row), fp32."""
    rng = np.random.default_rng(stable_seed(tag))
    g = rng.normal(0, 1, (rows, cols)) * np.exp(rng.normal(0, 1, (rows, 1)))
    return (g * g).astype(np.float32)


def check_split_sens(w, sens, ppm, top_ppm):
    got, arrays = split_sens_on_gpu(w, sens, ppm, top_ppm)
    t_min, t_max, t_s, nnz = q.split_thresholds(w, ppm, sens, top_ppm)
    assert got[0] == t_min and got[1] == t_max and got[3] == nnz
    assert got[2].view(np.uint32) == np.float32(t_s).view(np.uint32)
    want = q.extract(w, t_min, t_max, sens, t_s)
    for g, e in zip(arrays[:4], want):
        assert np.array_equal(g, e)
    assert np.array_equal(arrays[4].view(np.uint32), q.dense_sensitivity(sens, want[0], want[1]).view(np.uint32))
    return nnz


SPLIT_CASES = [(1, 1, 0), (1, 7, 250000), (37, 300, 2250), (130, 1000, 250), (130, 1000, 20000), (257, 4096, 2250),
               (64, 65536, 2250)]


@pytest.mark.parametrize("rows,cols,ppm", SPLIT_CASES)
def test_split_bit_exact(rows, cols, ppm):
    step(f"split rows={rows} cols={cols} ppm={ppm}")
    w = heavy(f"split{rows}x{cols}", rows, cols)
    got = split_on_gpu(w, ppm)
    t_min, t_max, nnz = q.thresholds(w, ppm)
    assert got[:3] == (t_min, t_max, nnz)
    rp, col, val, dense = q.extract(w, t_min, t_max)
    assert np.array_equal(got[3], rp)
    assert np.array_equal(got[4], col)
    assert np.array_equal(got[5], val)
    assert np.array_equal(got[6], dense)


def test_split_special_values():
    """Signed zeros, infinities, repeated values and a constant row."""
    step("split special values")
    w = heavy("special", 20, 512)
    w[0, :] = 0x3C00                       # constant row of 1.0
    w[1, :8] = [0x8000, 0x0000, 0x7C00, 0xFC00, 0x7BFF, 0xFBFF, 0x0001, 0x8001]
    w[2, ::2] = 0x8000
    for ppm in (0, 100, 2250, 100000):
        got = split_on_gpu(w, ppm)
        t_min, t_max, nnz = q.thresholds(w, ppm)
        assert got[:3] == (t_min, t_max, nnz)
        want = q.extract(w, t_min, t_max)
        for g, e in zip(got[3:], want):
            assert np.array_equal(g, e)
    # every value equal: both thresholds are that value and nothing is an outlier
    w1 = np.full((3, 300), 0xB400, np.uint16)
    assert split_on_gpu(w1, 2250)[:3] == (0xB400, 0xB400, 0)


def test_split_capacity_overflow_reported():
    step("split capacity")
    w = heavy("capacity", 65, 1024)
    t_min, t_max, nnz = q.thresholds(w, 20000)
    assert nnz > 10
    wd = u16_to_dev(w)
    with pytest.raises(nw().SqllmError) as e:
        nw().outlier_extract(wd, t_min, t_max, nnz - 1)
    assert e.value.status == 9
    rp, col, val, dense = nw().outlier_extract(wd, t_min, t_max, nnz)   # exactly enough
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_u16(col), q.extract(w, t_min, t_max)[1])


def test_split_full_layer_rank_property():
    """LLaMA-65B down projection (8192 x 22016) at 0.45% outliers (0.225%
    on each side): T_min / T_max hold their ranks in the total order, and
    W = D + S exactly with the oracle's CSR given those thresholds."""
    rows, cols, ppm = 8192, 22016, 2250
    w = heavy("full-split", rows, cols)
    step(f"split full rows={rows} cols={cols} ppm={ppm}")
    t_min, t_max, nnz, rp, col, val, dense = split_on_gpu(w, ppm)
    n = rows * cols
    tail = n * ppm // 1_000_000
    keys = q.total_order_key(w.ravel())
    k_lo, k_hi = q.total_order_key(np.array([t_min, t_max]))
    assert np.count_nonzero(keys < k_lo) <= tail < np.count_nonzero(keys <= k_lo)
    assert np.count_nonzero(keys > k_hi) <= tail < np.count_nonzero(keys >= k_hi)
    del keys
    want = q.extract(w, t_min, t_max)
    assert nnz == want[1].size
    assert 0.004 < nnz / n < 0.005
    for g, e in zip((rp, col, val, dense), want):
        assert np.array_equal(g, e)


@pytest.mark.parametrize("rows,cols,ppm,top_ppm", [(1, 9, 100000, 200000), (37, 300, 2000, 500),
                                                    (130, 1000, 2000, 5000), (257, 4096, 2000, 500),
                                                    (64, 65536, 2000, 500), (20, 512, 0, 0)])
def test_split_with_sensitivities_bit_exact(rows, cols, ppm, top_ppm):
    step(f"split+sens rows={rows} cols={cols} ppm={ppm} top={top_ppm}")
    w = heavy(f"splits{rows}x{cols}", rows, cols)
    sens = fisher_like(f"fisher{rows}x{cols}", rows, cols)
    check_split_sens(w, sens, ppm, top_ppm)


def test_split_sensitivity_order_and_ties():
    """Repeated sensitivities (ties at T_s stay dense), zeros, negative
    values and -0 (total order), and values that share their high 16 bits."""
    step("split+sens ties")
    rows, cols = 16, 640
    w = heavy("ties", rows, cols)
    rng = np.random.default_rng(stable_seed("ties-sens"))
    sens = rng.choice(np.array([0.0, 1.0, 2.0, 3.0], np.float32), (rows, cols))
    sens[3] = -rng.exponential(1.0, cols).astype(np.float32)
    sens[4, :10] = -0.0
    base = np.float32(5.0).view(np.uint32)
    sens[5] = (base + rng.integers(0, 4096, cols).astype(np.uint32)).view(np.float32)  # one high half
    for top in (0, 500, 20000, 300000):
        check_split_sens(w, sens, 2000, top)


def test_split_sensitivity_full_layer_rank_property():
    """LLaMA-65B down projection (8192 x 22016): 0.4% outliers (0.2 / 99.8
    percentiles) plus the 0.05% most sensitive weights, as on the pages;
    T_s holds its rank, S is the oracle's given the thresholds."""
    rows, cols, ppm, top = 8192, 22016, 2000, 500
    w = heavy("full-split", rows, cols)
    sens = fisher_like("full-fisher", rows, cols)
    step(f"split+sens full rows={rows} cols={cols}")
    got, arrays = split_sens_on_gpu(w, sens, ppm, top)
    t_min, t_max, t_s, nnz = got
    n = rows * cols
    n_top = n * top // 1_000_000
    keys = q.total_order_key32(sens.ravel().view(np.uint32))
    k_s = q.total_order_key32(np.array([t_s]).view(np.uint32))[0]
    assert np.count_nonzero(keys > k_s) <= n_top < np.count_nonzero(keys >= k_s)
    del keys
    want = q.extract(w, t_min, t_max, sens, t_s)
    assert nnz == want[1].size
    assert 0.0040 < nnz / n < 0.0046          # 0.4% + 0.05%, less the overlap
    for g, e in zip(arrays[:4], want):
        assert np.array_equal(g, e)


def kmeans_on_gpu(d, bits, iters, sens=None):
    sd = None if sens is None else torch.from_numpy(sens).cuda()
    codes, lut = nw().kmeans_lut(u16_to_dev(d), bits, iters, sd)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), dev_to_u16(lut)


KM_CASES = [(1, 7, 3, 20), (37, 300, 3, 20), (37, 300, 4, 0), (37, 300, 4, 1), (130, 1000, 4, 20),
            (65, 4096, 3, 30), (37, 300, 2, 20), (130, 1000, 2, 1)]


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("rows,cols,bits,iters", KM_CASES)
def test_kmeans_bit_exact(rows, cols, bits, iters, weighted):
    step(f"kmeans rows={rows} cols={cols} bits={bits} iters={iters} weighted={weighted}")
    d = heavy(f"km{rows}x{cols}", rows, cols)
    sens = None
    if weighted:
        rng = np.random.default_rng(stable_seed(f"sens{rows}x{cols}"))
        sens = rng.exponential(1.0, (rows, cols)).astype(np.float32)
        sens[0, :] = 0                     # a row without sensitivity keeps the uniform start
    codes, lut = kmeans_on_gpu(d, bits, iters, sens)
    want_codes, want_lut = q.kmeans_lut(d, sens, bits, iters)
    assert np.array_equal(lut, want_lut)
    assert np.array_equal(codes, want_codes)


def test_kmeans_on_split_dense_part():
    """k-means of D after the split (zeros where the outliers were)."""
    step("kmeans on dense part")
    w = heavy("km-split", 64, 2048)
    t_min, t_max, _ = q.thresholds(w, 2250)
    d = q.extract(w, t_min, t_max)[3]
    codes, lut = kmeans_on_gpu(d, 3, 20)
    want_codes, want_lut = q.kmeans_lut(d, None, 3, 20)
    assert np.array_equal(lut, want_lut)
    assert np.array_equal(codes, want_codes)


def test_kmeans_table_rounds_once_to_fp16():
    """A centroid just above the midpoint of two adjacent fp16 values must
    round up: rounding through fp32 first would land on the midpoint and
    then go to the even neighbour (below)."""
    step("kmeans fp16 rounding")
    a = int(np.float16(0.4285).view(np.uint16)) & ~1          # even significand
    b = a + 1
    row = np.array([[0xBC00, 0x3C00, a, b]], np.uint16)         # -1, 1, a, b
    sens = np.array([[1.0, 1.0, 1.0, 1.0 + 2.0 ** -17]], np.float32)
    codes, lut = kmeans_on_gpu(row, 3, 1, sens)
    want_codes, want_lut = q.kmeans_lut(row, sens, 3, 1)
    assert want_lut[0, 5] == b                                   # the oracle's single rounding
    assert np.array_equal(lut, want_lut)
    assert np.array_equal(codes, want_codes)


def test_kmeans_full_layer_sampled_rows():
    """LLaMA-65B query projection (8192 x 8192), 3-bit, weighted, 20 steps:
    every row computed on the GPU, 12 sampled rows (first, last, random)
    against the oracle."""
    rows, cols, bits, iters = 8192, 8192, 3, 20
    d = heavy("full-km", rows, cols)
    rng = np.random.default_rng(stable_seed("full-km-sens"))
    sens = rng.exponential(1.0, (rows, cols)).astype(np.float32)
    step(f"kmeans full rows={rows} cols={cols} bits={bits}")
    codes, lut = kmeans_on_gpu(d, bits, iters, sens)
    sample = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 10)]))
    want_codes, want_lut = q.kmeans_lut(d[sample], sens[sample], bits, iters)
    assert np.array_equal(lut[sample], want_lut)
    assert np.array_equal(codes[sample], want_codes)
    # all rows: the table is sorted and each code is the nearest entry
    lv = q.f16_to_f64(lut)
    assert np.all(np.diff(lv, axis=1) >= 0)
    x = q.f16_to_f64(d[:64])
    dist = np.abs(x[:, :, None] - lv[:64, None, :])
    assert np.array_equal(codes[:64], np.argmin(dist, axis=2))


def test_split_kmeans_pack_product_pipeline():
    """W -> thresholds -> CSR + D -> k-means -> pack -> (D_hat + S) x, every
    step on the GPU, against the oracle's own pipeline and product."""
    rows, cols, bits = 300, 1024, 3
    w = heavy("pipeline", rows, cols)
    x = np.random.default_rng(stable_seed("pipeline-x")).normal(0, 1, (2, cols)).astype(np.float16).view(np.uint16)
    step("pipeline split/kmeans/pack/product")
    wd = u16_to_dev(w)
    t_min, t_max, _, nnz = nw().outlier_thresholds(wd, 2250)
    rp, col, val, dense = nw().outlier_extract(wd, t_min, t_max, nnz)
    codes, lut = nw().kmeans_lut(dense, bits, 20)
    packed = nw().pack(codes, bits)
    y = nw().dense_sparse_gemv(packed, lut, bits, rp, col, val, u16_to_dev(x))
    torch.cuda.synchronize()
    o_min, o_max, _ = q.thresholds(w, 2250)
    o_rp, o_col, o_val, o_dense = q.extract(w, o_min, o_max)
    o_codes, o_lut = q.kmeans_lut(o_dense, None, bits, 20)
    assert np.array_equal(codes.cpu().numpy(), o_codes)
    y_ref, scale = oracle.dense_sparse_gemv(o_codes, o_lut, bits, o_rp, o_col, o_val, x)
    assert_close(y, y_ref, scale, what="pipeline")


def test_weighted_pipeline_with_sensitive_values():
    """The pages' full recipe on one layer: 0.4% outliers + 0.05% sensitive
    values to S, D clustered with its sensitivities (zero at S), 4-bit,
    packed and multiplied, against the oracle's own pipeline."""
    rows, cols, bits = 260, 2048, 4
    w = heavy("wpipe", rows, cols)
    sens = fisher_like("wpipe-fisher", rows, cols)
    x = np.random.default_rng(stable_seed("wpipe-x")).normal(0, 1, (3, cols)).astype(np.float16).view(np.uint16)
    step("weighted pipeline")
    wd, sd = u16_to_dev(w), torch.from_numpy(sens).cuda()
    t_min, t_max, t_s, nnz = nw().outlier_thresholds(wd, 2000, sd, 500)
    rp, col, val, dense, sdense = nw().outlier_extract(wd, t_min, t_max, nnz, sd, t_s)
    codes, lut = nw().kmeans_lut(dense, bits, 25, sdense)
    packed = nw().pack(codes, bits)
    y = nw().dense_sparse_gemv(packed, lut, bits, rp, col, val, u16_to_dev(x))
    torch.cuda.synchronize()
    o_min, o_max, o_s, _ = q.split_thresholds(w, 2000, sens, 500)
    o_rp, o_col, o_val, o_dense = q.extract(w, o_min, o_max, sens, o_s)
    o_codes, o_lut = q.kmeans_lut(o_dense, q.dense_sensitivity(sens, o_rp, o_col), bits, 25)
    assert np.array_equal(dev_to_u16(lut), o_lut)
    assert np.array_equal(codes.cpu().numpy(), o_codes)
    y_ref, scale = oracle.dense_sparse_gemv(o_codes, o_lut, bits, o_rp, o_col, o_val, x)
    assert_close(y, y_ref, scale, what="weighted pipeline")


def test_two_bit_pipeline_with_a_tenth_percent_sparse():
    """The pages' 2-bit setting (Appendix F, Tables F.8 / F.10): 0.05%
    outliers (0.025% per tail) plus 0.05% sensitive values to S, four
    weighted centroids per row, packed and multiplied, against the oracle's
    own pipeline."""
    rows, cols, bits = 300, 2048, 2
    w = heavy("twobit", rows, cols)
    sens = fisher_like("twobit-fisher", rows, cols)
    x = np.random.default_rng(stable_seed("twobit-x")).normal(0, 1, (2, cols)).astype(np.float16).view(np.uint16)
    step("2-bit pipeline")
    wd, sd = u16_to_dev(w), torch.from_numpy(sens).cuda()
    t_min, t_max, t_s, nnz = nw().outlier_thresholds(wd, 250, sd, 500)
    rp, col, val, dense, sdense = nw().outlier_extract(wd, t_min, t_max, nnz, sd, t_s)
    codes, lut = nw().kmeans_lut(dense, bits, 25, sdense)
    packed = nw().pack(codes, bits)
    y = nw().dense_sparse_gemv(packed, lut, bits, rp, col, val, u16_to_dev(x))
    torch.cuda.synchronize()
    o_min, o_max, o_s, o_nnz = q.split_thresholds(w, 250, sens, 500)
    assert nnz == o_nnz and 0.0009 < nnz / (rows * cols) < 0.0011
    o_rp, o_col, o_val, o_dense = q.extract(w, o_min, o_max, sens, o_s)
    o_codes, o_lut = q.kmeans_lut(o_dense, q.dense_sensitivity(sens, o_rp, o_col), bits, 25)
    assert np.array_equal(dev_to_u16(lut), o_lut)
    assert np.array_equal(codes.cpu().numpy(), o_codes)
    y_ref, scale = oracle.dense_sparse_gemv(o_codes, o_lut, bits, o_rp, o_col, o_val, x)
    assert_close(y, y_ref, scale, 5e-3, what="2-bit pipeline")
