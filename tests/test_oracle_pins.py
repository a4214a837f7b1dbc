"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Every check here compares the oracle with something it does not compute
itself: numpy's IEEE binary16 conversions over all bit patterns, hand-derived
bytes of the packed layout (tests/golden/layout_cases.json), a packer written
here with Python integers from the layout definition, a brute-force product
over an explicitly materialised weight matrix (numpy fp16 decoding + numpy
matmul), scipy.sparse CSR products, closed forms (constant and affine lookup
tables, one-hot activations) and exact integer arithmetic.  Between them a
dropped dense or sparse term, a wrong sign, a swapped LUT index, a transposed
operand or a misplaced byte fails at least one test; test_planted_mistakes
shows it by compiling deliberately broken copies of the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.sparse as sp

import oracle
from seeds import stable_seed
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- binary16

def test_f16_decoder_matches_numpy_on_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_array_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _halfway_points(rng, n):
    """Exact midpoints between adjacent finite fp16 values (ties)."""
    h = rng.integers(0, 0x7BFF, n).astype(np.uint16)  # h and h+1 both finite, positive
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0
    return np.concatenate([mid, -mid])


def test_f16_encoder_matches_numpy_round_to_nearest_even():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        _halfway_points(rng, 5000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf]),
    ])
    ours = oracle.f64_array_to_f16(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- layout

def _golden():
    with open(os.path.join(GOLD, "layout_cases.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_unpack_hand_derived_bytes(case):
    bits, rows, cols = case["bits"], case["rows"], case["cols"]
    buf = np.zeros(oracle.packed_bytes(rows, cols, bits), dtype=np.uint8)
    for off, val in case["bytes"]:
        buf[off] = val
    want = np.zeros((rows, cols), dtype=np.uint8)
    for r, c, code in case["codes"]:
        want[r, c] = code
    assert np.array_equal(oracle.unpack(buf, rows, cols, bits), want)


@pytest.mark.parametrize("pat", _golden()["patterns"], ids=lambda c: c["name"])
def test_unpack_hand_derived_patterns(pat):
    bits, rows, cols = pat["bits"], pat["rows"], pat["cols"]
    buf = np.zeros(oracle.packed_bytes(rows, cols, bits), dtype=np.uint8)
    for q, hx in enumerate(pat["pieces_hex"]):
        buf[1024 * q:1024 * q + 16] = np.frombuffer(bytes.fromhex(hx), dtype=np.uint8)
    got = oracle.unpack(buf, rows, cols, bits)
    want = (np.arange(cols) % (1 << bits)).astype(np.uint8)[None, :]
    assert np.array_equal(got, want)


def test_packed_bytes_formula():
    # 64-row tiles, exactly b bits per code
    assert oracle.packed_bytes(130, 512, 3) == 3 * 64 * 512 * 3 // 8
    assert oracle.packed_bytes(64, 256, 4) == 64 * 256 // 2
    assert oracle.packed_bytes(22016, 8192, 3) == 22016 * 8192 * 3 // 8
    assert oracle.packed_bytes(65, 512, 2) == 2 * 64 * 512 // 4


def group_string(codes_row_group: np.ndarray, bits: int) -> bytes:
    """The 32*bits-byte string of one (row, 256-column group), from the layout
    definition: pairs p = code[2p] | code[2p+1] << bits; 4-bit: byte p is
    pair p; 2-bit: byte p holds pair 2p in its low and pair 2p+1 in its high
    four bits; 3-bit: units of 12 bytes / 16 pairs, pair p < 12 in the low six
    bits of unit byte p, pair 12+q spread two bits at a time over the top two
    bits of unit bytes q, 4+q, 8+q."""
    c = [int(v) for v in codes_row_group]
    pairs = [c[2 * p] | (c[2 * p + 1] << bits) for p in range(128)]
    if bits == 4:
        return bytes(pairs)
    if bits == 2:
        return bytes(pairs[2 * p] | (pairs[2 * p + 1] << 4) for p in range(64))
    out = bytearray(96)
    for u in range(8):
        unit = pairs[16 * u:16 * u + 16]
        for p in range(12):
            out[12 * u + p] |= unit[p]
        for q in range(4):
            for k in range(3):
                out[12 * u + 4 * k + q] |= ((unit[12 + q] >> (2 * k)) & 3) << 6
    return bytes(out)


def pack_from_definition(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packer written here from the layout definition (Python integers)."""
    rows, cols = codes.shape
    T, G, P = (rows + 63) // 64, cols // 256, 2 * bits
    buf = np.zeros(T * G * P * 1024, dtype=np.uint8)
    for r in range(rows):
        t, l = divmod(r, 64)
        for g in range(G):
            string = group_string(codes[r, 256 * g:256 * g + 256], bits)
            for q in range(P):
                off = ((t * G + g) * P + q) * 1024 + l * 16
                buf[off:off + 16] = np.frombuffer(string[16 * q:16 * q + 16], dtype=np.uint8)
    return buf


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(1, 256), (63, 512), (65, 256), (130, 768)])
def test_unpack_roundtrip_with_independent_packer(bits, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols + bits)
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    assert np.array_equal(oracle.unpack(pack_from_definition(codes, bits), rows, cols, bits), codes)


# ---------------------------------------------------------------- product

def _f16(a):
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


def _rand_f16(rng, shape, sigma):
    return (rng.standard_normal(shape) * sigma).astype(np.float16).view(np.uint16)


def _csr_from_mask(rng, mask, sigma=0.2):
    rows, cols = mask.shape
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(mask.sum(axis=1))
    r_idx, c_idx = np.nonzero(mask)
    col = c_idx.astype(np.uint16)
    val = _rand_f16(rng, col.size, sigma)
    return row_ptr, col, val


def _what(codes, lut, row_ptr, col, val):
    """Explicit reconstructed weights: numpy fp16 decode, fancy-index gather,
    CSR scattered by scipy."""
    W = np.take_along_axis(_f16(lut), codes.astype(np.int64), axis=1)
    if row_ptr is not None and col.size:
        S = sp.csr_matrix((_f16(val), col.astype(np.int64), row_ptr.astype(np.int64)), shape=W.shape)
        W = W + S.toarray()
    return W


SPARSITY = ["none", "one", "5pct", "50pct", "full", "empty_rows", "dense_row"]


def _make_case(rng, rows, cols, bits, batch, sparsity):
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    lut = _rand_f16(rng, (rows, 1 << bits), 0.02)
    x = _rand_f16(rng, (batch, cols), 1.0)
    if sparsity == "none":
        mask = np.zeros((rows, cols), bool)
    elif sparsity == "one":
        mask = np.zeros((rows, cols), bool)
        mask[rng.integers(rows), rng.integers(cols)] = True
    elif sparsity == "5pct":
        mask = rng.random((rows, cols)) < 0.05
    elif sparsity == "50pct":
        mask = rng.random((rows, cols)) < 0.5
    elif sparsity == "full":
        mask = np.ones((rows, cols), bool)
    elif sparsity == "empty_rows":
        mask = rng.random((rows, cols)) < 0.05
        mask[::2] = False
    else:  # one fully dense row, the rest sparse
        mask = rng.random((rows, cols)) < 0.01
        mask[rows // 2] = True
    rp, col, val = _csr_from_mask(rng, mask)
    return codes, lut, x, rp, col, val


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols,batch", [(1, 256, 1), (2, 512, 3), (7, 768, 8), (65, 256, 2), (257, 512, 1)])
@pytest.mark.parametrize("sparsity", SPARSITY)
def test_product_matches_brute_force(bits, rows, cols, batch, sparsity):
    rng = np.random.default_rng(stable_seed(bits, rows, cols, batch, sparsity))
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, sparsity)
    y, s = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    W = _what(codes, lut, rp, col, val)
    X = _f16(x)
    y_bf = X @ W.T
    s_bf = np.abs(X) @ np.abs(W).T
    assert y.shape == (batch, rows)
    assert np.all(np.abs(y - y_bf) <= 1e-12 * s_bf + 1e-300)
    assert np.allclose(s, s_bf, rtol=1e-12, atol=0)


def test_selected_rows_match_full_product():
    rng = np.random.default_rng(7)
    codes, lut, x, rp, col, val = _make_case(rng, 130, 512, 3, 2, "5pct")
    y, s = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    sel = np.array([129, 0, 64, 77])
    ys, ss = oracle.dense_sparse_gemv(codes[sel], lut, 3, rp, col, val, x, rows=130, sel=sel)
    assert np.array_equal(ys, y[:, sel]) and np.array_equal(ss, s[:, sel])


def test_no_outliers_equals_dense_only():
    rng = np.random.default_rng(8)
    codes, lut, x, _, _, _ = _make_case(rng, 65, 512, 4, 2, "none")
    y0, s0 = oracle.dense_sparse_gemv(codes, lut, 4, None, None, None, x)
    rp = np.zeros(66, np.int32)
    y1, s1 = oracle.dense_sparse_gemv(codes, lut, 4, rp, np.zeros(0, np.uint16), np.zeros(0, np.uint16), x)
    assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


def test_constant_lut_closed_form():
    """LUT[r][:] = v_r  =>  y_r = v_r * sum(x)  (no outliers)."""
    rng = np.random.default_rng(9)
    rows, cols = 33, 768
    v = _rand_f16(rng, rows, 0.05)
    lut = np.repeat(v[:, None], 8, axis=1)
    codes = rng.integers(0, 8, (rows, cols)).astype(np.uint8)
    x = _rand_f16(rng, (1, cols), 1.0)
    y, _ = oracle.dense_sparse_gemv(codes, lut, 3, None, None, None, x)
    sx = math.fsum(_f16(x)[0])
    assert np.allclose(y[0], _f16(v) * sx, rtol=1e-13, atol=1e-15)


def test_affine_lut_closed_form():
    """Uniform quantisation as the special case of the lookup table:
    LUT[r][j] = a_r + j d_r  =>  y_r = a_r sum(x) + d_r sum_c code[r][c] x_c."""
    rng = np.random.default_rng(10)
    rows, cols, bits = 20, 512, 4
    a = rng.integers(-64, 64, rows) / 1024.0
    d = rng.integers(1, 16, rows) / 4096.0
    lut_f = a[:, None] + np.arange(16)[None, :] * d[:, None]
    lut = lut_f.astype(np.float16).view(np.uint16)
    assert np.array_equal(_f16(lut), lut_f)  # exactly representable
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    x = _rand_f16(rng, (1, cols), 1.0)
    X = _f16(x)[0]
    y, _ = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    want = np.array([a[r] * math.fsum(X) + d[r] * math.fsum(codes[r] * X) for r in range(rows)])
    assert np.allclose(y[0], want, rtol=1e-12, atol=1e-14)


def test_single_code_plus_sparse_closed_form():
    """All codes equal j  =>  y_r = LUT[r][j] sum(x) + (S x)_r (scipy CSR)."""
    rng = np.random.default_rng(11)
    rows, cols = 40, 512
    codes = np.full((rows, cols), 5, np.uint8)
    lut = _rand_f16(rng, (rows, 8), 0.02)
    rp, col, val = _csr_from_mask(rng, rng.random((rows, cols)) < 0.05)
    x = _rand_f16(rng, (1, cols), 1.0)
    X = _f16(x)[0]
    S = sp.csr_matrix((_f16(val), col.astype(np.int64), rp.astype(np.int64)), shape=(rows, cols))
    y, _ = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    want = _f16(lut)[:, 5] * math.fsum(X) + S @ X
    assert np.allclose(y[0], want, rtol=1e-12, atol=1e-14)


def test_one_hot_activation_returns_a_weight_column():
    """x = e_c  =>  y = What[:, c] = LUT[r][code[r][c]] + S[r][c]."""
    rng = np.random.default_rng(12)
    rows, cols = 70, 256
    codes, lut, _, rp, col, val = _make_case(rng, rows, cols, 3, 1, "50pct")
    S = sp.csr_matrix((_f16(val), col.astype(np.int64), rp.astype(np.int64)), shape=(rows, cols)).toarray()
    for c in (0, 17, 255):
        x = np.zeros((1, cols), np.uint16)
        x[0, c] = 0x3C00  # 1.0
        y, s = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        want = _f16(lut)[np.arange(rows), codes[:, c]] + S[:, c]
        assert np.array_equal(y[0], want)
        assert np.array_equal(s[0], np.abs(want))


def test_zero_lut_is_plain_csr_spmv():
    rng = np.random.default_rng(13)
    rows, cols = 100, 768
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    lut = np.zeros((rows, 16), np.uint16)
    rp, col, val = _csr_from_mask(rng, rng.random((rows, cols)) < 0.1)
    x = _rand_f16(rng, (3, cols), 1.0)
    S = sp.csr_matrix((_f16(val), col.astype(np.int64), rp.astype(np.int64)), shape=(rows, cols))
    y, _ = oracle.dense_sparse_gemv(codes, lut, 4, rp, col, val, x)
    want = (S @ _f16(x).T).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-14)


def test_integer_inputs_are_exact():
    """Small-integer LUT, x and outliers: the fp64 result equals the exact
    integer sum (Python integers)."""
    rng = np.random.default_rng(14)
    rows, cols, bits, batch = 9, 512, 3, 2
    lut_i = rng.integers(-2, 3, (rows, 8))
    x_i = rng.integers(-2, 3, (batch, cols))
    mask = rng.random((rows, cols)) < 0.1
    rp, col, _ = _csr_from_mask(rng, mask)
    val_i = rng.integers(-4, 5, col.size)
    codes = rng.integers(0, 8, (rows, cols)).astype(np.uint8)
    lut = lut_i.astype(np.float16).view(np.uint16)
    x = x_i.astype(np.float16).view(np.uint16)
    val = val_i.astype(np.float16).view(np.uint16)
    y, _ = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    for b in range(batch):
        for r in range(rows):
            exact = sum(int(lut_i[r, codes[r, c]]) * int(x_i[b, c]) for c in range(cols))
            exact += sum(int(val_i[i]) * int(x_i[b, col[i]]) for i in range(rp[r], rp[r + 1]))
            assert y[b, r] == exact


def test_normaliser_equals_result_for_nonnegative_inputs():
    rng = np.random.default_rng(15)
    rows, cols = 30, 256
    codes = rng.integers(0, 8, (rows, cols)).astype(np.uint8)
    lut = np.abs(_f16(_rand_f16(rng, (rows, 8), 0.02))).astype(np.float16).view(np.uint16)
    x = np.abs(_f16(_rand_f16(rng, (2, cols), 1.0))).astype(np.float16).view(np.uint16)
    rp, col, val = _csr_from_mask(rng, rng.random((rows, cols)) < 0.05)
    val = np.abs(_f16(val)).astype(np.float16).view(np.uint16)
    y, s = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    assert np.allclose(y, s, rtol=1e-13, atol=0)


def test_spmv_add_matches_scipy():
    rng = np.random.default_rng(16)
    rows, cols, batch = 90, 512, 4
    rp, col, val = _csr_from_mask(rng, rng.random((rows, cols)) < 0.03)
    x = _rand_f16(rng, (batch, cols), 1.0)
    y_in = _rand_f16(rng, (batch, rows), 0.5)
    S = sp.csr_matrix((_f16(val), col.astype(np.int64), rp.astype(np.int64)), shape=(rows, cols))
    y, s = oracle.spmv_add(rp, col, val, x, y_in, rows)
    want = _f16(y_in) + (S @ _f16(x).T).T
    want_s = np.abs(_f16(y_in)) + (abs(S) @ np.abs(_f16(x)).T).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-14)
    assert np.allclose(s, want_s, rtol=1e-12, atol=1e-14)


def test_decode_is_lut_gather():
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 16, (5, 256)).astype(np.uint8)
    lut = rng.integers(0, 65536, (5, 16)).astype(np.uint16)
    w = oracle.decode(codes, lut, 4)
    assert np.array_equal(w, lut[np.arange(5)[:, None], codes])


def test_tolerance_rule():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    scale = np.array([[10.0, 10.0, 0.0]])
    good = np.array([[1.04, -2.04, 0.0]], np.float16).view(np.uint16)
    ok, worst = oracle.within_tolerance(good, y_ref, scale)
    assert ok and worst < 5e-3
    bad = np.array([[1.1, -2.0, 0.0]], np.float16).view(np.uint16)
    assert not oracle.within_tolerance(bad, y_ref, scale)[0]
    nonzero = np.array([[1.0, -2.0, 1e-3]], np.float16).view(np.uint16)
    assert not oracle.within_tolerance(nonzero, y_ref, scale)[0]


def test_on_generated_workload_shapes():
    """Oracle on a generator-made 0.45% layer equals the brute force."""
    spec = synth.MatrixSpec("t", 130, 512, 3, batch=2)
    m = synth.make_matrix(spec, seed=0, workload=99)
    y, s = oracle.dense_sparse_gemv(m.codes, m.lut, 3, m.row_ptr, m.col, m.val, m.x)
    W = _what(m.codes, m.lut, m.row_ptr, m.col, m.val)
    X = _f16(m.x)
    assert np.all(np.abs(y - X @ W.T) <= 1e-12 * (np.abs(X) @ np.abs(W).T))
