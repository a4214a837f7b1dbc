"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: packing (against a packer written from the layout definition),
unpacking, decoding, integer-valued products.  Floating point: every output
within 5e-3 of the oracle's fp64 result, normalised by sum |W||x| of its row
(rows where the normaliser is 0 must be exactly 0).  Sizes span several
64-row tiles, several 256-column groups and ragged row tails.
"""
import numpy as np
import pytest
import torch

import oracle
from seeds import stable_seed
import synth
from gpu_util import DevMatrix, assert_close, dev_to_u16, nw, step, u16_to_dev
from test_oracle_pins import _make_case, _rand_f16, pack_from_definition

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _f16(a):
    return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)


# ------------------------------------------------------------ pack / unpack

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(1, 256), (63, 512), (65, 256), (130, 768), (257, 1024)])
def test_pack_bytes_equal_definition(bits, rows, cols):
    step(f"pack bits={bits} rows={rows} cols={cols}")
    rng = np.random.default_rng(rows + cols + bits)
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    packed = nw().pack(torch.from_numpy(codes).cuda(), bits)
    torch.cuda.synchronize()
    want = pack_from_definition(codes, bits)
    assert packed.numel() == want.size == oracle.packed_bytes(rows, cols, bits)
    assert np.array_equal(packed.cpu().numpy(), want)
    # the oracle reads the GPU's bytes back to the same codes
    assert np.array_equal(oracle.unpack(packed.cpu().numpy(), rows, cols, bits), codes)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(1, 256), (65, 768), (300, 2048)])
def test_unpack_and_decode_bit_exact(bits, rows, cols):
    step(f"unpack/decode bits={bits} rows={rows} cols={cols}")
    rng = np.random.default_rng(7 * rows + cols + bits)
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    # tables with subnormals, signed zeros, the largest finite values
    lut = rng.integers(0, 0x7C00, (rows, 1 << bits)).astype(np.uint16) | (rng.integers(0, 2, (rows, 1 << bits)) << 15).astype(np.uint16)
    lut[:, 0] = 0x8000
    lut[:, 1] = 0x0001
    lut[0, :] = 0x7BFF
    packed = nw().pack(torch.from_numpy(codes).cuda(), bits)
    got_codes = nw().unpack_codes(packed, rows, cols, bits)
    got_w = nw().decode_weights(packed, u16_to_dev(lut), rows, cols, bits)
    torch.cuda.synchronize()
    assert np.array_equal(got_codes.cpu().numpy(), codes)
    assert np.array_equal(dev_to_u16(got_w), oracle.decode(codes, lut, bits))


def test_pack_rejects_out_of_range_code():
    step("pack code range")
    codes = np.zeros((64, 256), np.uint8)
    codes[10, 100] = 8
    with pytest.raises(nw().SqllmError) as e:
        nw().pack(torch.from_numpy(codes).cuda(), 3)
    assert e.value.status == 6
    codes[10, 100] = 16
    with pytest.raises(nw().SqllmError):
        nw().pack(torch.from_numpy(codes).cuda(), 4)
    codes[10, 100] = 15
    nw().pack(torch.from_numpy(codes).cuda(), 4)


# ------------------------------------------------------------ products, small shapes

SHAPES = [(1, 256, 1), (7, 768, 3), (65, 512, 2), (130, 2048, 1), (257, 1024, 8), (300, 4096, 1), (129, 1024, 16),
          (64, 22016, 2)]
SPARSITY = ["none", "one", "5pct", "50pct", "full", "empty_rows", "dense_row"]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols,batch", SHAPES)
@pytest.mark.parametrize("sparsity", SPARSITY)
def test_fused_matches_oracle(bits, rows, cols, batch, sparsity):
    step(f"fused bits={bits} rows={rows} cols={cols} batch={batch} sparsity={sparsity}")
    rng = np.random.default_rng(stable_seed(bits, rows, cols, batch, sparsity))
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, sparsity)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y = d.fused()
    torch.cuda.synchronize()
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    assert_close(y, y_ref, scale, TOL, "fused")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rows,cols,batch", SHAPES)
def test_gemv_matches_oracle(bits, rows, cols, batch):
    step(f"gemv bits={bits} rows={rows} cols={cols} batch={batch}")
    rng = np.random.default_rng(stable_seed(bits, rows, cols, batch, "gemv"))
    codes, lut, x, _, _, _ = _make_case(rng, rows, cols, bits, batch, "none")
    d = DevMatrix(codes, lut, bits, None, None, None, x)
    y = d.gemv()
    torch.cuda.synchronize()
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    assert_close(y, y_ref, scale, TOL, "gemv")


@pytest.mark.parametrize("rows,cols,batch", SHAPES)
@pytest.mark.parametrize("sparsity", ["one", "5pct", "full", "empty_rows", "dense_row"])
def test_spmv_add_matches_oracle(rows, cols, batch, sparsity):
    step(f"spmv_add rows={rows} cols={cols} batch={batch} sparsity={sparsity}")
    rng = np.random.default_rng(stable_seed(rows, cols, batch, sparsity, "spmv"))
    _, _, x, rp, col, val = _make_case(rng, rows, cols, 3, batch, sparsity)
    y_in = (rng.standard_normal((batch, rows)) * 0.5).astype(np.float16).view(np.uint16)
    codes = np.zeros((rows, cols), np.uint8)
    d = DevMatrix(codes, np.zeros((rows, 8), np.uint16), 3, rp, col, val, x)
    y = u16_to_dev(y_in.copy())
    d.spmv_add(y)
    torch.cuda.synchronize()
    y_ref, scale = oracle.spmv_add(rp, col, val, x, y_in, rows)
    assert_close(y, y_ref, scale, TOL, "spmv_add")


def test_spmv_add_without_outliers_is_noop():
    step("spmv_add nnz=0")
    rows, cols = 70, 512
    x = u16_to_dev(np.zeros((1, cols), np.uint16))
    y0 = (np.arange(rows, dtype=np.float64) / 7).astype(np.float16).view(np.uint16)[None, :]
    y = u16_to_dev(y0.copy())
    nw().spmv_add(torch.zeros(rows + 1, dtype=torch.int32, device="cuda"), None, None, x, y)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_u16(y), y0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_stream_ordered_pair_equals_fused(bits):
    step(f"gemv+spmv_add vs fused bits={bits}")
    rng = np.random.default_rng(31 + bits)
    rows, cols, batch = 257, 2048, 2
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, "5pct")
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y2 = d.gemv()
    d.spmv_add(y2)
    y1 = d.fused()
    torch.cuda.synchronize()
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    assert_close(y1, y_ref, scale, TOL, "fused")
    assert_close(y2, y_ref, scale, TOL, "stream-ordered")


def _integer_case(rng, rows, cols, bits, batch, dense_max=2, sparse_max=4, density=0.05):
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    lut = rng.integers(-dense_max, dense_max + 1, (rows, 1 << bits)).astype(np.float16).view(np.uint16)
    x = rng.integers(-2, 3, (batch, cols)).astype(np.float16).view(np.uint16)
    mask = rng.random((rows, cols)) < density
    rp = np.zeros(rows + 1, np.int32)
    rp[1:] = np.cumsum(mask.sum(axis=1))
    col = np.nonzero(mask)[1].astype(np.uint16)
    val = rng.integers(-sparse_max, sparse_max + 1, col.size).astype(np.float16).view(np.uint16)
    return codes, lut, x, rp, col, val


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("rows,cols,batch", [(65, 768, 1), (300, 4096, 3), (130, 22016, 1)])
def test_integer_inputs_bit_exact(bits, rows, cols, batch):
    """Integer LUT, x and outliers: every fp32 partial sum is an exact integer,
    so the single fp16 rounding of the fused call is determined."""
    step(f"integer fused bits={bits} rows={rows} cols={cols} batch={batch}")
    rng = np.random.default_rng(rows * cols + bits)
    codes, lut, x, rp, col, val = _integer_case(rng, rows, cols, bits, batch)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y = d.fused()
    yg = d.gemv()
    torch.cuda.synchronize()
    y_ref, _ = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    assert np.array_equal(dev_to_u16(y), oracle.f64_array_to_f16(y_ref))
    yd_ref, _ = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    assert np.array_equal(dev_to_u16(yg), oracle.f64_array_to_f16(yd_ref))


@pytest.mark.parametrize("bits", [3, 4])
def test_integer_stream_ordered_bit_exact(bits):
    """With |D x| <= 2048 the intermediate fp16 is exact, so gemv followed by
    spmv_add rounds to the same bits as the fused call."""
    step(f"integer stream-ordered bits={bits}")
    rng = np.random.default_rng(5 + bits)
    rows, cols, batch = 200, 256, 2
    codes, lut, x, rp, col, val = _integer_case(rng, rows, cols, bits, batch, dense_max=2, density=0.1)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y = d.gemv()
    d.spmv_add(y)
    yf = d.fused()
    torch.cuda.synchronize()
    y_ref, _ = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    want = oracle.f64_array_to_f16(y_ref)
    assert np.array_equal(dev_to_u16(y), want)
    assert np.array_equal(dev_to_u16(yf), want)


def test_subnormal_inputs_are_not_flushed():
    """Tables of fp16 subnormals times small-integer activations: exact
    results of a few units of 2^-24, which a flush to zero would lose."""
    step("subnormals")
    rng = np.random.default_rng(77)
    rows, cols, bits = 130, 512, 3
    codes = rng.integers(0, 8, (rows, cols)).astype(np.uint8)
    lut = rng.integers(0, 4, (rows, 8)).astype(np.uint16)  # 0..3 units of 2^-24
    lut |= (rng.integers(0, 2, (rows, 8)) << 15).astype(np.uint16)
    x = np.zeros((1, cols), np.uint16)
    x[0, rng.choice(cols, 6, replace=False)] = np.float16(1.0).view(np.uint16)
    d = DevMatrix(codes, lut, bits, None, None, None, x)
    y = d.fused()
    torch.cuda.synchronize()
    y_ref, _ = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    assert np.any(y_ref != 0)
    assert np.array_equal(dev_to_u16(y), oracle.f64_array_to_f16(y_ref))


def test_batch_equals_separate_calls():
    """A batch of 8 gives each column what a batch-1 call gives it, up to the
    fp32 summation order (batch 1 spreads its sums over more accumulators):
    every column of both is within the parity bound of the oracle and the two
    differ by at most one fp16 ulp."""
    step("batch 8 vs 8 x batch 1")
    rng = np.random.default_rng(3)
    rows, cols, bits = 257, 2048, 3
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, 8, "5pct")
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y8 = d.fused()
    singles = []
    for b in range(8):
        db = DevMatrix(codes, lut, bits, rp, col, val, x[b:b + 1])
        singles.append(db.fused())
    torch.cuda.synchronize()
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    assert_close(y8, y_ref, scale, TOL, "batch 8")
    y8 = dev_to_u16(y8)
    for b in range(8):
        assert_close(singles[b], y_ref[b:b + 1], scale[b:b + 1], TOL, f"batch 1, column {b}")
        one = dev_to_u16(singles[b])[0]
        ulps = np.abs(y8[b].view(np.int16).astype(np.int64) - one.view(np.int16).astype(np.int64))
        same_sign = (y8[b] >> 15) == (one >> 15)
        assert np.all(ulps[same_sign] <= 1), f"column {b}: batch 8 and batch 1 differ by {ulps.max()} ulp"


def test_repeated_calls_are_bit_identical():
    step("determinism")
    rng = np.random.default_rng(4)
    codes, lut, x, rp, col, val = _make_case(rng, 300, 4096, 3, 2, "dense_row")
    d = DevMatrix(codes, lut, 3, rp, col, val, x)
    outs = [dev_to_u16(d.fused()) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("rows,cols,bits,zipf", [(4096, 11008, 4, False), (5120, 13824, 3, True)])
@pytest.mark.parametrize("batch", [1, 6])
def test_split_combine_is_deterministic(rows, cols, bits, zipf, batch):
    """Down projections of LLaMA-7B and LLaMA-13B run split over many
    workgroups per row tile; their partial sums meet in a fixed binary tree,
    so repeated calls, with one workspace or another, give identical bits
    whichever workgroup ends first."""
    spec = synth.MatrixSpec("down", rows, cols, bits, batch, 45, zipf)
    (plan,), _ = nw().launch_plan([(rows, cols, spec.nnz)], batch=batch)
    assert plan["split"] > 1 or plan["slice_tiles"] > 0
    step(f"determinism {rows}x{cols} bits {bits} batch {batch} plan {plan}")
    m = synth.make_matrix(spec, seed=0, workload=2 if rows == 4096 else 3, index=1 if rows == 4096 else 6)
    d = DevMatrix.from_synth(m)
    ws2 = torch.zeros(nw().workspace_bytes(rows, cols, batch), dtype=torch.uint8, device="cuda")
    outs = [dev_to_u16(d.fused()) for _ in range(4)] + [dev_to_u16(d.fused(ws=ws2)) for _ in range(2)]
    for k, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"call {k} differs in {int((outs[0] != o).sum())} outputs"
    assert int(ws2.view(torch.int32).abs().sum().item()) == 0
    sel = np.sort(np.random.default_rng(stable_seed("det", rows, batch)).choice(rows, 512, replace=False))
    y_ref, scale = oracle.dense_sparse_gemv(m.codes[sel], m.lut, bits, m.row_ptr, m.col, m.val, m.x, rows=rows,
                                            sel=sel)
    ok, worst = oracle.within_tolerance(outs[0][:, sel], y_ref, scale, TOL)
    assert ok, f"max normalised error {worst:.3e}"


def test_two_streams_default_workspaces():
    """Calls without a workspace on two streams at once: each stream gets
    its own cached workspace, and both results match the oracle."""
    step("two streams, default workspaces")
    rng = np.random.default_rng(12)
    cases = [_make_case(rng, 4096, 8192, 3, 1, "5pct"), _make_case(rng, 8192, 4096, 3, 6, "5pct")]
    mats = [DevMatrix(codes, lut, 3, rp, col, val, x) for codes, lut, x, rp, col, val in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    ys = [[], []]
    for _ in range(3):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                ys[k].append(mats[k].fused())
    torch.cuda.synchronize()
    for k in range(2):
        codes, lut, x, rp, col, val = cases[k]
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        for y in ys[k]:
            assert_close(y, y_ref, scale, TOL, f"stream {k}")


@pytest.mark.parametrize("kib", [1, 5, 4095, 4096 * 9 + 7])
def test_stream_read_reads_every_word_once(kib):
    """The reference read stream behind the ceiling measurement reads each
    32-bit word exactly once: its XOR equals numpy's (ragged ranges, fewer
    pieces than waves, a tail on the last wave)."""
    rng = np.random.default_rng(kib)
    words = rng.integers(0, 2 ** 32, kib * 256, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((4096,), -1, dtype=torch.int32, device="cuda")
    step(f"stream read {kib} KiB")
    nw().stream_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert int(np.bitwise_xor.reduce(got)) == int(np.bitwise_xor.reduce(words))


def test_permuted_table_with_remapped_codes():
    """Permuting a row's table entries together with its codes leaves y unchanged."""
    step("lut permutation invariance")
    rng = np.random.default_rng(9)
    rows, cols, bits = 130, 1024, 4
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, 1, "5pct")
    perm = rng.permutation(16)
    inv = np.argsort(perm)
    lut2 = lut[:, perm]          # entry j of the new table = old entry perm[j]
    codes2 = inv[codes].astype(np.uint8)
    y1 = DevMatrix(codes, lut, bits, rp, col, val, x).fused()
    y2 = DevMatrix(codes2, lut2, bits, rp, col, val, x).fused()
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_u16(y1), dev_to_u16(y2))


def test_workspace_shared_across_shapes():
    """One workspace serves consecutive calls of different shapes on a stream."""
    step("workspace reuse")
    rng = np.random.default_rng(10)
    ws = torch.zeros(nw().workspace_bytes(22016, 8192, 2), dtype=torch.uint8, device="cuda")
    cases = []
    for rows, cols, batch in [(4096, 8192, 1), (130, 2048, 2), (22016, 8192, 1), (1000, 4096, 1), (8192, 4096, 2),
                              (22016, 4096, 1)]:
        codes, lut, x, rp, col, val = _make_case(rng, rows, cols, 3, batch, "5pct")
        d = DevMatrix(codes, lut, 3, rp, col, val, x)
        cases.append((d.fused(ws=ws), codes, lut, x, rp, col, val))
    torch.cuda.synchronize()
    for y, codes, lut, x, rp, col, val in cases:
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, "shared workspace")
    # every (sum, count) word was reset by the workgroup that completed it
    assert int(ws.view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("split,waves", [(1, 1), (1, 12), (1, 16), (2, 8), (3, 5), (3, 12), (7, 2), (16, 1), (0, 0)])
def test_launch_configurations(bits, split, waves):
    """Column splits and waves per workgroup of every kind give the same
    answer (one wave per workgroup included)."""
    step(f"launch config bits={bits} split={split} waves={waves}")
    rng = np.random.default_rng(waves * 100 + split + bits)
    rows, cols, batch = 193, 4096, 2
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, "dense_row")
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    try:
        nw().set_tuning(split=split, waves=waves)
        y = d.fused()
        yg = d.gemv()
        ys = d.spmv_add(yg.clone())
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    assert_close(y, y_ref, scale, TOL, "fused")
    assert_close(ys, y_ref, scale, TOL, "stream-ordered")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("form", ["matrix", "dot"])
def test_dense_forms_every_batch(bits, batch, form):
    """Both forms of the dense part -- the matrix-core form (the default) and
    the v_dot2c form -- at every batch, fused and dense-only, with
    16 waves (x staged in LDS for the outliers, beside the pair table and the
    waves' x slots), 8 and 3 waves (outliers read x from global memory)."""
    rng = np.random.default_rng(stable_seed(bits, batch, form, "forms"))
    rows, cols = 193, 4096
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, "5pct")
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    yd_ref, dscale = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    for waves in (16, 8, 3):
        step(f"dense form={form} bits={bits} batch={batch} waves={waves}")
        try:
            nw().set_tuning(waves=waves, dot_only=1 if form == "dot" else 0)
            y = d.fused()
            yg = d.gemv()
            torch.cuda.synchronize()
        finally:
            nw().set_tuning()
        assert_close(y, y_ref, scale, TOL, f"fused waves={waves}")
        assert_close(yg, yd_ref, dscale, TOL, f"gemv waves={waves}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("batch", [9, 12, 16])
def test_matrix_form_above_batch_8(bits, batch):
    """Batches 9-16 (matrix-core form only: three or four batch quads on the
    same weight operand), fused and dense-only, 16 / 8 / 3 waves."""
    rng = np.random.default_rng(stable_seed(bits, batch, "above-8"))
    rows, cols = 193, 4096
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, "5pct")
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    yd_ref, dscale = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    for waves in (16, 8, 3):
        step(f"matrix form bits={bits} batch={batch} waves={waves}")
        try:
            nw().set_tuning(waves=waves)
            y = d.fused()
            yg = d.gemv()
            torch.cuda.synchronize()
        finally:
            nw().set_tuning()
        assert_close(y, y_ref, scale, TOL, f"fused waves={waves}")
        assert_close(yg, yd_ref, dscale, TOL, f"gemv waves={waves}")


# ------------------------------------------------------------ the evaluation workloads

def _check_matrix(m: synth.Matrix, sel=None, ws=None):
    d = DevMatrix.from_synth(m)
    y = d.fused(ws=ws)
    torch.cuda.synchronize()
    if sel is None:
        y_ref, scale = oracle.dense_sparse_gemv(m.codes, m.lut, m.spec.bits, m.row_ptr, m.col, m.val, m.x)
        return assert_close(y, y_ref, scale, TOL, m.spec.name)
    sel = np.asarray(sel)
    y_ref, scale = oracle.dense_sparse_gemv(m.codes[sel], m.lut, m.spec.bits, m.row_ptr, m.col, m.val, m.x,
                                            rows=m.spec.rows, sel=sel)
    return assert_close(y[:, torch.from_numpy(sel).cuda()], y_ref, scale, TOL, m.spec.name)


@pytest.mark.parametrize("workload", [1, 2, 3])
def test_workload_full(workload):
    for i, spec in enumerate(synth.workload(workload)):
        step(f"workload {workload} matrix {i} {spec}")
        m = synth.make_matrix(spec, seed=0, workload=workload, index=i)
        _check_matrix(m)


@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16])
def test_workload4(batch):
    """The three LLaMA-65B shapes at every batch: every output against the oracle."""
    for i, spec in enumerate(synth.workload(4, batch=batch)):
        step(f"workload 4 batch {batch} matrix {i} {spec}")
        m = synth.make_matrix(spec, seed=0, workload=4, index=i)
        _check_matrix(m)


@pytest.mark.parametrize("bits,density_bp", [(3, 0), (3, 5), (3, 45), (4, 0), (4, 5), (4, 45)])
def test_workload5_layer_sample(bits, density_bp):
    """The 80-layer stream at full size: its last layer's 7 linears (the
    stream's matrix indices 553..559, as the benchmark draws them), one
    workspace shared by all calls as in the benchmark, every row of each
    checked against the oracle."""
    specs = synth.workload(5, bits=bits, density_bp=density_bp)
    ws = torch.zeros(nw().workspace_bytes(22016, 22016, 1), dtype=torch.uint8, device="cuda")
    for i in range(len(specs) - 7, len(specs)):
        spec = specs[i]
        step(f"workload 5 bits {bits} density {density_bp}bp matrix {i} {spec}")
        m = synth.make_matrix(spec, seed=0, workload=5, index=i)
        assert m.col.size == spec.nnz
        _check_matrix(m, ws=ws)


def test_graph_replay_matches_eager():
    """The benchmark times HIP-graph replays of the fused call: a captured
    sequence of calls sharing one workspace gives, on every replay, the bits
    of the same calls made eagerly."""
    specs = [synth.MatrixSpec("q", 8192, 8192, 3), synth.MatrixSpec("gate", 22016, 8192, 3),
             synth.MatrixSpec("down", 8192, 22016, 3), synth.MatrixSpec("small", 4096, 4096, 4, 1, 5)]
    ws = torch.zeros(nw().workspace_bytes(22016, 22016, 1), dtype=torch.uint8, device="cuda")
    mats = []
    for i, spec in enumerate(specs):
        step(f"graph replay: prepare {spec}")
        mats.append(DevMatrix.from_synth(synth.make_matrix(spec, seed=3, workload=5, index=i)))
    eager = [d.fused(ws=ws) for d in mats]
    torch.cuda.synchronize()
    eager = [dev_to_u16(y) for y in eager]
    outs = [torch.empty((1, d.rows), dtype=torch.float16, device="cuda") for d in mats]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    step("graph replay: capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for d, y in zip(mats, outs):
                d.fused(y=y, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        step(f"graph replay {rep}")
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (y, ref) in enumerate(zip(outs, eager)):
            assert np.array_equal(dev_to_u16(y), ref), f"replay {rep} matrix {k} differs from the eager call"


# ------------------------------------------------------------ several products in one launch

def _items(mats, ys):
    return [dict(packed=d.packed, lut=d.lut, row_ptr=d.row_ptr, col=d.col, val=d.val, x=d.x, y=y)
            for d, y in zip(mats, ys)]


GROUP_CASES = [(193, 4096, "5pct"), (64, 256, "none"), (1000, 2048, "empty_rows"), (7, 768, "full"),
               (300, 8192, "one"), (129, 512, "dense_row")]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("batch", [1, 3, 8, 16])
def test_group_matches_oracle(bits, batch):
    """Products of different shapes, with and without outliers (two launches),
    ragged row tails: each output within tolerance of the oracle."""
    rng = np.random.default_rng(stable_seed("group", bits, batch))
    cases = [_make_case(rng, r, c, bits, batch, sp) for r, c, sp in GROUP_CASES]
    mats = [DevMatrix(*case[:2], bits, *case[3:], case[2]) for case in cases]
    ys = [torch.full((batch, d.rows), float("nan"), dtype=torch.float16, device="cuda") for d in mats]
    step(f"group bits {bits} batch {batch}: {GROUP_CASES}")
    nw().dense_sparse_gemv_group(_items(mats, ys), bits)
    torch.cuda.synchronize()
    for (codes, lut, x, rp, col, val), y, shape in zip(cases, ys, GROUP_CASES):
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, f"group item {shape}")


def _plan_dev(row_ptr):
    plan = nw().outlier_plan(row_ptr)
    return torch.from_numpy(plan).cuda(), int(plan[0])


def _heavy_tiles_case(rng, rows, cols, bits, batch, heavy_rows):
    """Sparse rows (1%) plus a few fully dense rows, so that their tiles hold
    far more nonzeros than the rest."""
    codes = rng.integers(0, 1 << bits, (rows, cols)).astype(np.uint8)
    lut = _rand_f16(rng, (rows, 1 << bits), 0.02)
    x = _rand_f16(rng, (batch, cols), 1.0)
    mask = rng.random((rows, cols)) < 0.01
    mask[list(heavy_rows)] = True
    r, c = np.nonzero(mask)
    rp = np.zeros(rows + 1, np.int32)
    np.add.at(rp, r + 1, 1)
    rp = np.cumsum(rp).astype(np.int32)
    return codes, lut, x, rp, c.astype(np.uint16), _rand_f16(rng, (r.size,), 0.5)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("batch", [1, 3, 6, 16])
def test_outlier_plan_heavy_tiles(bits, batch):
    """Tiles with fully dense rows get helper workgroups from the outlier
    plan: every output within tolerance of the oracle (the ragged last tile
    heavy too), repeated calls bit-identical, the workspace zero again."""
    rng = np.random.default_rng(stable_seed("plan", bits, batch))
    rows, cols = 4000, 4096
    codes, lut, x, rp, col, val = _heavy_tiles_case(rng, rows, cols, bits, batch, (70, 71, 72, 600, 3998, 3999))
    plan, h = _plan_dev(rp)
    assert h > 0
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    ws = torch.zeros(nw().workspace_bytes(rows, cols, batch), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y = torch.full((batch, rows), float("nan"), dtype=torch.float16, device="cuda")
        step(f"planned heavy tiles bits {bits} batch {batch} helpers {h}")
        nw().dense_sparse_gemv_group([dict(packed=d.packed, lut=d.lut, row_ptr=d.row_ptr, col=d.col, val=d.val,
                                           x=d.x, y=y, plan=plan)], bits, ws=ws)
        torch.cuda.synchronize()
        outs.append(dev_to_u16(y))
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    ok, worst = oracle.within_tolerance(outs[0], y_ref, scale, TOL)
    assert ok, f"max normalised error {worst:.3e}"
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert int(ws.view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("index", [0, 4, 6])
@pytest.mark.parametrize("batch", [1, 6])
def test_outlier_plan_13b_zipf(index, batch):
    """The 13B layer's products with Zipf rows (the skewed workload), planned:
    every row against the oracle, bit-identical repeats."""
    s = synth.workload(3)[index]
    spec = synth.MatrixSpec(s.name, s.rows, s.cols, s.bits, batch, s.density_bp, s.zipf)
    m = synth.make_matrix(spec, seed=0, workload=3, index=index)
    plan, h = _plan_dev(m.row_ptr)
    assert h > 0
    d = DevMatrix.from_synth(m)
    step(f"planned 13B {spec.name} batch {batch} helpers {h}")
    item = dict(packed=d.packed, lut=d.lut, row_ptr=d.row_ptr, col=d.col, val=d.val, x=d.x, plan=plan,
                plan_helpers=h)
    outs = []
    for _ in range(2):
        y = torch.full((batch, spec.rows), float("nan"), dtype=torch.float16, device="cuda")
        nw().dense_sparse_gemv_group([dict(item, y=y)], spec.bits)
        torch.cuda.synchronize()
        outs.append(dev_to_u16(y))
    assert np.array_equal(outs[0], outs[1])
    y_ref, scale = oracle.dense_sparse_gemv(m.codes, m.lut, spec.bits, m.row_ptr, m.col, m.val, m.x)
    ok, worst = oracle.within_tolerance(outs[0], y_ref, scale, TOL)
    assert ok, f"max normalised error {worst:.3e}"


@pytest.mark.parametrize("split", [0, 1, 3, 8])
def test_outlier_plan_in_mixed_groups(split):
    """A group mixing a planned product, an unplanned one, a plan without
    helpers and a product without outliers, at default and forced splits
    (owners plus helpers up to 16 partial sums per tile)."""
    rng = np.random.default_rng(stable_seed("plan-mixed", split))
    bits, batch = 3, 2
    cases = [_heavy_tiles_case(rng, 300, 2048, bits, batch, (5, 6, 290)),
             _make_case(rng, 193, 4096, bits, batch, "5pct"),
             _make_case(rng, 130, 1024, bits, batch, "5pct"),
             _make_case(rng, 64, 256, bits, batch, "none")]
    mats = [DevMatrix(*c[:2], bits, *c[3:], c[2]) for c in cases]
    ys = [torch.full((batch, d.rows), float("nan"), dtype=torch.float16, device="cuda") for d in mats]
    items = _items(mats, ys)
    items[0]["plan"], h0 = _plan_dev(cases[0][3])
    items[2]["plan"], h2 = _plan_dev(cases[2][3])
    assert h0 > 0 and h2 == 0
    step(f"planned mixed group split {split} helpers {h0}")
    try:
        nw().set_tuning(split=split)
        nw().dense_sparse_gemv_group(items, bits)
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    for (codes, lut, x, rp, col, val), y in zip(cases, ys):
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, f"mixed planned group, split {split}")


@pytest.mark.parametrize("batch", [1, 5])
def test_group_of_eight_products(batch):
    """The most products a group call takes (8): with and without outliers
    mixed (two launches), ragged shapes, distinct x; each matches the oracle."""
    rng = np.random.default_rng(stable_seed("group-eight", batch))
    shapes = [(193, 4096, "5pct"), (64, 256, "none"), (300, 2048, "none"), (1000, 1024, "empty_rows"),
              (7, 768, "full"), (129, 512, "dense_row"), (65, 8192, "one"), (257, 1024, "none")]
    cases = [_make_case(rng, r, c, 3, batch, sp) for r, c, sp in shapes]
    mats = []
    for (r, c, sp), (codes, lut, x, rp, col, val) in zip(shapes, cases):
        if sp == "none":
            rp = col = val = None
        mats.append(DevMatrix(codes, lut, 3, rp, col, val, x))
    ys = [torch.full((batch, d.rows), float("nan"), dtype=torch.float16, device="cuda") for d in mats]
    step(f"group of eight batch {batch}")
    nw().dense_sparse_gemv_group(_items(mats, ys), 3)
    torch.cuda.synchronize()
    for (r, c, sp), (codes, lut, x, rp, col, val), y in zip(shapes, cases, ys):
        if sp == "none":
            rp = col = val = None
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, f"group item {r}x{c} {sp}")


def test_group_graph_replay_matches_eager():
    """Group launches captured in a HIP graph give, on every replay, the bits
    of the same launches made eagerly: a layer's (q, k, v) (two workgroups per
    unit, q at split 2) and (gate, up) at batch 1, and a batch-6 group whose
    products share one x (its transposed copy is written and cleared by
    kernels inside the graph).  Eager calls run between the replays."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    specs = synth.workload(5, bits=3, density_bp=45)[:7]
    groups = []
    for level in ([0, 1, 2], [4, 5]):
        ms = [synth.make_matrix(specs[i], seed=5, workload=5, index=i) for i in level]
        groups.append(([DevMatrix.from_synth(m) for m in ms], 1))
    rng = np.random.default_rng(stable_seed("group-graph"))
    x6 = (rng.standard_normal((6, 4096))).astype(np.float16).view(np.uint16)
    mats6 = []
    for k in range(3):
        codes, lut, _, rp, col, val = _make_case(rng, 1024, 4096, 3, 6, "50pct")
        d = DevMatrix(codes, lut, 3, rp, col, val, x6)
        mats6.append(d)
    shared = mats6[0].x
    for d in mats6:
        d.x = shared
    groups.append((mats6, 6))
    step("group graph: eager")
    eager = []
    for mats, batch in groups:
        ys = [torch.empty((batch, d.rows), dtype=torch.float16, device="cuda") for d in mats]
        nw().dense_sparse_gemv_group(_items(mats, ys), 3, ws=ws)
        eager.append(ys)
    torch.cuda.synchronize()
    eager = [[dev_to_u16(y) for y in ys] for ys in eager]
    outs = [[torch.empty((batch, d.rows), dtype=torch.float16, device="cuda") for d in mats] for mats, batch in groups]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    step("group graph: capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for (mats, batch), ys in zip(groups, outs):
                nw().dense_sparse_gemv_group(_items(mats, ys), 3, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        step(f"group graph replay {rep}")
        for ys in outs:
            for y in ys:
                y.fill_(float("nan"))
        mats6[1].fused(ws=ws)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for gi, (ys, refs) in enumerate(zip(outs, eager)):
            for k, (y, ref) in enumerate(zip(ys, refs)):
                assert np.array_equal(dev_to_u16(y), ref), f"replay {rep} group {gi} product {k} differs"
    assert int(ws.view(torch.int32).abs().sum().item()) == 0, "workspace not zero after the replays"


@pytest.mark.parametrize("split", [1, 2])
def test_group_equals_single_calls(split):
    """With the launch shape fixed, a product computed inside a group has the
    bits of the same product computed alone."""
    rng = np.random.default_rng(stable_seed("group-single", split))
    cases = [_make_case(rng, r, c, 3, 2, sp) for r, c, sp in GROUP_CASES]
    mats = [DevMatrix(*case[:2], 3, *case[3:], case[2]) for case in cases]
    try:
        nw().set_tuning(split=split, waves=8)
        ys = [torch.empty((2, d.rows), dtype=torch.float16, device="cuda") for d in mats]
        step(f"group vs single, split {split}")
        nw().dense_sparse_gemv_group(_items(mats, ys), 3)
        singles = [d.fused() for d in mats]
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    for y, ys_, shape in zip(ys, singles, GROUP_CASES):
        assert np.array_equal(dev_to_u16(y), dev_to_u16(ys_)), f"group item {shape} differs from the single call"


@pytest.mark.parametrize("bits,batch,sparsity", [(3, 1, "5pct"), (3, 3, "dense_row"), (4, 6, "50pct"),
                                                   (2, 2, "none"), (3, 16, "5pct")])
def test_row_slices_for_two_slots(bits, batch, sparsity):
    """A product of more row tiles than compute units but fewer than twice as
    many runs as two row slices in one launch, the first at split 2.  Rows
    on both sides of the slice boundary, the ragged last tile and a random
    sample match the oracle; repeated calls give the same bits; the unsliced
    launch (forced split 1, or a workspace without room for the first
    slice's words) matches the oracle too."""
    rng = np.random.default_rng(stable_seed("row-slices", bits, batch, sparsity))
    rows, cols = 64 * 300 + 17, 4096  # 301 tiles: 211 at split 2, then 90 whole (the last ragged)
    boundary = 211 * 64
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, sparsity)
    if sparsity == "none":
        rp = col = val = None
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    sel = np.unique(np.concatenate([[0, 63, 64, boundary - 65, boundary - 64, boundary - 1, boundary, boundary + 1,
                                     boundary + 63, boundary + 64, rows - 17, rows - 1],
                                    rng.choice(rows, 1500, replace=False)]))
    y_ref, scale = oracle.dense_sparse_gemv(codes[sel], lut, bits, rp, col, val, x, rows=rows, sel=sel)
    sel_dev = torch.from_numpy(sel).cuda()
    step(f"row slices bits={bits} batch={batch} {sparsity}")
    y1 = d.fused()
    y2 = d.fused()
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_u16(y1), dev_to_u16(y2)), "repeated sliced calls differ"
    assert_close(y1[:, sel_dev], y_ref, scale, TOL, "sliced")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    y3 = d.fused(ws=small)
    try:
        nw().set_tuning(split=1)
        y4 = d.fused()
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    assert_close(y3[:, sel_dev], y_ref, scale, TOL, "unsliced (small workspace)")
    assert_close(y4[:, sel_dev], y_ref, scale, TOL, "unsliced (forced split 1)")
    if sparsity != "none":
        yd = d.gemv()
        torch.cuda.synchronize()
        yd_ref, dscale = oracle.dense_sparse_gemv(codes[sel], lut, bits, None, None, None, x, rows=rows, sel=sel)
        assert_close(yd[:, sel_dev], yd_ref, dscale, TOL, "sliced dense-only")


# ------------------------------------------------------------ the compact 3-bit pair table

# (rows, cols, batch, sparsity): x fits in LDS beside the compact table but not
# beside the full one -- one workgroup per compute unit at batch 8, 4 and 2,
# and 301 row tiles (two row slices, two workgroups per unit) at batch 4
COMPACT_CASES = [(300, 8192, 8, "5pct"), (200, 16384, 4, "dense_row"), (130, 32768, 2, "5pct"),
                 (64 * 300 + 17, 4096, 4, "empty_rows")]


@pytest.mark.parametrize("rows,cols,batch,sparsity", COMPACT_CASES)
def test_compact_table_launches(rows, cols, batch, sparsity):
    """Fused 3-bit launches that stage x beside the compact pair table (the
    64 pair entries once, addressed with the top two bits of each address byte
    cleared): every row within tolerance of the oracle, repeated calls give
    the same bits, and integer inputs give exactly the fp16 rounding of the
    oracle's result."""
    (plan,), _ = nw().launch_plan([(rows, cols, 1)], batch=batch)
    assert plan["compact"] == 1 and plan["xt"] == 0
    rng = np.random.default_rng(stable_seed("compact", rows, cols, batch, sparsity))
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, 3, batch, sparsity)
    d = DevMatrix(codes, lut, 3, rp, col, val, x)
    step(f"compact table rows={rows} cols={cols} batch={batch} {sparsity}")
    y1 = d.fused()
    y2 = d.fused()
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_u16(y1), dev_to_u16(y2)), "repeated calls differ"
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    assert_close(y1, y_ref, scale, TOL, f"compact {rows}x{cols} batch {batch}")
    step(f"compact table, integer inputs rows={rows} cols={cols} batch={batch}")
    codes, lut, x, rp, col, val = _integer_case(rng, rows, cols, 3, batch)
    d = DevMatrix(codes, lut, 3, rp, col, val, x)
    y = d.fused()
    torch.cuda.synchronize()
    y_ref, _ = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    assert np.array_equal(dev_to_u16(y), oracle.f64_array_to_f16(y_ref))


def test_compact_table_group():
    """A group launch takes the compact table for all its products when one
    of them needs it to stage x; a product whose x would fit either way, and
    one without outliers (its own launch, full table), still match."""
    rng = np.random.default_rng(stable_seed("compact-group"))
    batch = 8
    shapes = [(300, 8192, "5pct"), (129, 2048, "dense_row"), (64, 4096, "none")]
    plans, _ = nw().launch_plan([(r, c, 0 if sp == "none" else 1) for r, c, sp in shapes], batch=batch, mode=1)
    assert all(p["compact"] == 1 for p in plans)
    cases = [_make_case(rng, r, c, 3, batch, sp) for r, c, sp in shapes]
    cases = [(co, lu, xx, None, None, None) if sp == "none" else (co, lu, xx, rp, cl, va)
             for (co, lu, xx, rp, cl, va), (_, _, sp) in zip(cases, shapes)]
    mats = [DevMatrix(*case[:2], 3, *case[3:], case[2]) for case in cases]
    ys = [torch.full((batch, d.rows), float("nan"), dtype=torch.float16, device="cuda") for d in mats]
    step(f"compact group batch {batch}: {shapes}")
    nw().dense_sparse_gemv_group(_items(mats, ys), 3)
    torch.cuda.synchronize()
    for (codes, lut, x, rp, col, val), y, shape in zip(cases, ys, shapes):
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, f"compact group item {shape}")


@pytest.mark.parametrize("batch", [4, 6, 8])
def test_group_shared_x(batch):
    """Products that share one x (as q, k and v do) share one transposed copy
    of it for their outliers (at batch >= 5: their 600K+ nonzeros pass the
    threshold); the product with another x (fewer nonzeros) reads x in place."""
    rng = np.random.default_rng(stable_seed("group-shared-x", batch))
    cols = 4096
    x = (rng.standard_normal((batch, cols))).astype(np.float16).view(np.uint16)
    x2 = (rng.standard_normal((batch, cols))).astype(np.float16).view(np.uint16)
    shapes = [(300, "50pct", x), (129, "dense_row", x), (64, "full", x2), (193, "one", x)]
    cases = []
    for rows, sp, xx in shapes:
        codes, lut, _, rp, col, val = _make_case(rng, rows, cols, 3, batch, sp)
        cases.append((codes, lut, xx, rp, col, val))
    xd, x2d = u16_to_dev(x), u16_to_dev(x2)
    mats = [DevMatrix(c[0], c[1], 3, c[3], c[4], c[5], c[2]) for c in cases]
    for d, (_, _, xx) in zip(mats, shapes):
        d.x = xd if xx is x else x2d                 # one device copy per distinct x
    ys = [torch.full((batch, d.rows), float("nan"), dtype=torch.float16, device="cuda") for d in mats]
    step(f"group shared x batch {batch}")
    nw().dense_sparse_gemv_group(_items(mats, ys), 3)
    torch.cuda.synchronize()
    for (codes, lut, xx, rp, col, val), y, (rows, sp, _) in zip(cases, ys, shapes):
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, xx)
        assert_close(y, y_ref, scale, TOL, f"group item {rows} {sp}")


def test_one_workspace_many_shapes():
    """One workspace serves calls of different shapes and batches in any
    order: after each call (transposed x included: the batch 8 and 6 calls
    carry over 400K nonzeros) it is all zero again."""
    rng = np.random.default_rng(stable_seed("ws-many"))
    seq = [(300, 4096, 8, "50pct"), (1000, 2048, 1, "5pct"), (64, 8192, 6, "full"), (2000, 256, 2, "one"),
           (129, 4096, 3, "dense_row"), (200, 4096, 16, "50pct")]
    need = max(nw().workspace_bytes(r, c, b) for r, c, b, _ in seq)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rows, cols, batch, sp in seq + seq[::-1]:
        codes, lut, x, rp, col, val = _make_case(rng, rows, cols, 3, batch, sp)
        d = DevMatrix(codes, lut, 3, rp, col, val, x)
        step(f"shared workspace {rows}x{cols} batch {batch} {sp}")
        try:
            nw().set_tuning(split=2, waves=8)
            y = d.fused(ws=ws)
            torch.cuda.synchronize()
        finally:
            nw().set_tuning()
        y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
        assert_close(y, y_ref, scale, TOL, f"{rows}x{cols} batch {batch}")
        assert int(ws.count_nonzero().item()) == 0


@pytest.mark.parametrize("batch", [5, 8, 16])
def test_outliers_without_room_for_transposed_x(batch):
    """A workspace that holds only the (sum, count) words: the outliers read
    x in place; with the full workspace they read the transposed copy (526K
    nonzeros, over the threshold)."""
    rng = np.random.default_rng(stable_seed("no-xt", batch))
    rows, cols = 257, 4096
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, 3, batch, "50pct")
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    d = DevMatrix(codes, lut, 3, rp, col, val, x)
    words = -(-rows // 64) * 64 * batch * 8
    assert nw().workspace_bytes(rows, cols, batch) > words
    small = torch.zeros(words, dtype=torch.uint8, device="cuda")
    full = torch.zeros(nw().workspace_bytes(rows, cols, batch), dtype=torch.uint8, device="cuda")
    step(f"outliers without transposed x, batch {batch}")
    try:
        nw().set_tuning(split=2, waves=8)           # split: the words are needed; 8 waves: x not in LDS
        y_small = d.fused(ws=small)
        y_full = d.fused(ws=full)
        ys_small = d.spmv_add(d.gemv(ws=small), ws=small)
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    assert_close(y_small, y_ref, scale, TOL, "fused, words only")
    assert_close(y_full, y_ref, scale, TOL, "fused, full workspace")
    assert_close(ys_small, y_ref, scale, TOL, "stream-ordered, words only")


@pytest.mark.parametrize("density_bp", [0, 45])
def test_group_workload_levels(density_bp):
    """The stream's layer at full size in the launch groups the benchmark
    uses: (q, k, v) and (gate, up) in one launch each, 2048 sampled rows per
    product against the oracle."""
    specs = synth.workload(5, bits=3, density_bp=density_bp)[:7]
    rng = np.random.default_rng(stable_seed("group-levels", density_bp))
    for level in ([0, 1, 2], [4, 5]):
        ms = [synth.make_matrix(specs[i], seed=0, workload=5, index=i) for i in level]
        mats = [DevMatrix.from_synth(m) for m in ms]
        ys = [torch.empty((1, d.rows), dtype=torch.float16, device="cuda") for d in mats]
        step(f"group level {level} density {density_bp}bp")
        nw().dense_sparse_gemv_group(_items(mats, ys), 3)
        torch.cuda.synchronize()
        for m, y in zip(ms, ys):
            sel = np.sort(rng.choice(m.spec.rows, 2048, replace=False))
            y_ref, scale = oracle.dense_sparse_gemv(m.codes[sel], m.lut, 3, m.row_ptr, m.col, m.val, m.x,
                                                    rows=m.spec.rows, sel=sel)
            assert_close(y[:, torch.from_numpy(sel).cuda()], y_ref, scale, TOL, f"group {m.spec.name}")



# ------------------------------------------------------------ outlier ablation

@pytest.mark.parametrize("batch", [1, 3])
@pytest.mark.parametrize("sparsity", ["5pct", "dense_row", "empty_rows"])
def test_unbalanced_outlier_form_matches_oracle(batch, sparsity):
    """The ablation's one-thread-per-row outlier form gives the same product
    (within tolerance) as the balanced form, fused and outlier-only."""
    rng = np.random.default_rng(stable_seed("naive", batch, sparsity))
    codes, lut, x, rp, col, val = _make_case(rng, 193, 4096, 3, batch, sparsity)
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, 3, rp, col, val, x)
    d = DevMatrix(codes, lut, 3, rp, col, val, x)
    try:
        nw().set_tuning(sparse_naive=1)
        step(f"unbalanced outliers batch {batch} {sparsity}")
        y = d.fused()
        ys = d.spmv_add(d.gemv())
        torch.cuda.synchronize()
    finally:
        nw().set_tuning()
    assert_close(y, y_ref, scale, TOL, "fused, unbalanced outliers")
    assert_close(ys, y_ref, scale, TOL, "stream-ordered, unbalanced outliers")


def test_unbalanced_outlier_form_skewed_workload_rows():
    """The 13B layer's Zipf-skewed down projection (rows holding every
    column), sampled rows, unbalanced form."""
    spec = synth.workload(3)[6]
    m = synth.make_matrix(spec, seed=0, workload=3, index=6)
    try:
        nw().set_tuning(sparse_naive=1)
        step(f"unbalanced outliers {spec}")
        _check_matrix(m, np.arange(0, spec.rows, 7))
    finally:
        nw().set_tuning()


# ------------------------------------------------------------ the widest rows

@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("batch", [1, 9])
def test_maximum_columns(bits, batch):
    """cols = 65536, the most that 16-bit column indices address: x is then
    too wide to stage in LDS, so the outliers gather it from memory (from
    batch 5 on, from the transposed copy).  Nonzeros sit in the first and the
    last column, and the rows end in a ragged tile.  The fused, dense-only,
    stream-ordered, group and allocation-free calls all match the oracle."""
    rows, cols = 65, 65536
    rng = np.random.default_rng(stable_seed("maxcols", bits, batch))
    codes, lut, x, rp, col, val = _make_case(rng, rows, cols, bits, batch, "5pct")
    col = col.copy()
    assert rp[1] > rp[0] and rp[rows] > rp[rows - 1]
    col[rp[0]] = cols - 1      # row 0: a nonzero in the last column
    col[rp[rows] - 1] = 0      # last row: a nonzero in the first column
    d = DevMatrix(codes, lut, bits, rp, col, val, x)
    y_ref, scale = oracle.dense_sparse_gemv(codes, lut, bits, rp, col, val, x)
    yd_ref, sd = oracle.dense_sparse_gemv(codes, lut, bits, None, None, None, x)
    step(f"maximum columns bits={bits} batch={batch} nnz={col.size}")
    y_fused = d.fused()
    y_dense = d.gemv()
    y_pair = d.gemv()
    d.spmv_add(y_pair)
    y_group = torch.full((batch, rows), float("nan"), dtype=torch.float16, device="cuda")
    nw().dense_sparse_gemv_group(_items([d], [y_group]), bits)
    y_noalloc = torch.full((batch, rows), float("nan"), dtype=torch.float16, device="cuda")
    nw().dense_sparse_gemv_noalloc(d.packed, d.lut, bits, d.row_ptr, d.col, d.val, d.x, y_noalloc)
    torch.cuda.synchronize()
    assert_close(y_fused, y_ref, scale, TOL, "fused")
    assert_close(y_dense, yd_ref, sd, TOL, "dense only")
    assert_close(y_pair, y_ref, scale, TOL, "stream-ordered")
    assert_close(y_group, y_ref, scale, TOL, "group")
    assert np.array_equal(dev_to_u16(y_noalloc), dev_to_u16(y_fused)), "allocation-free call differs from the fused call"
