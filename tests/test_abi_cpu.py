"""The C ABI without a GPU: the library loads, exports every call that
include/sqllm.h declares, and rejects bad arguments on the host before any
HIP call.  Also the bytes accounting that the throughput figures use."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def nwpkg():
    import non_uniform_weight_amd
    return non_uniform_weight_amd


@pytest.fixture(scope="module")
def lib(nwpkg):
    return nwpkg.library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sqllm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sqllm_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib, nwpkg):
    names = declared_functions()
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(nwpkg.EXPORTS)


def test_status_strings(lib):
    for code in range(11):
        assert lib.sqllm_status_string(code).startswith(b"SQLLM_")
    assert lib.sqllm_status_string(99) == b"SQLLM_ERR_UNKNOWN"


def test_size_queries(nwpkg):
    assert nwpkg.packed_bytes(130, 512, 3) == 3 * 64 * 512 * 3 // 8
    assert nwpkg.packed_bytes(1, 256, 4) == 64 * 256 // 2
    assert nwpkg.packed_bytes(64, 100, 3) == 0
    assert nwpkg.packed_bytes(64, 256, 5) == 0
    assert nwpkg.packed_bytes(0, 256, 3) == 0
    assert nwpkg.packed_bytes(65, 512, 2) == 2 * 64 * 512 // 4
    assert nwpkg.packed_bytes(64, 256, 1) == 0
    assert nwpkg.workspace_bytes(22016, 8192, 1) >= 344 * 4
    assert nwpkg.workspace_bytes(22016, 8192, 17) == 0
    # combine words of the largest split (16 workgroups per row tile: 15 words
    # per output), then at batch >= 5 x transposed to [cols][8] ([cols][16] above 8)
    W15 = 15 * 64 * 8
    assert nwpkg.workspace_bytes(64, 8192, 12) == 12 * W15 + 8192 * 16 * 2
    assert nwpkg.workspace_bytes(100, 256, 1) == 2 * W15
    assert nwpkg.workspace_bytes(100, 256, 2) == 2 * 2 * W15
    assert nwpkg.workspace_bytes(100, 256, 4) == 2 * 4 * W15
    assert nwpkg.workspace_bytes(100, 256, 8) == 2 * 8 * W15 + 256 * 8 * 2
    assert nwpkg.workspace_bytes(64, 8192, 5) == 5 * W15 + 8192 * 8 * 2


P = ctypes.c_void_p
A16 = P(0x100000)        # fake, 256-byte aligned device addresses: never dereferenced
B16 = P(0x200000)
MIS = P(0x200002)


def gemv(lib, packed=A16, lut=B16, bits=3, rows=64, cols=256, x=A16, batch=1, y=B16, ws=A16, wsb=1 << 20):
    return lib.sqllm_gemv(packed, lut, bits, rows, cols, x, batch, y, ws, wsb, None)


def fused(lib, rp=A16, col=A16, val=A16, nnz=10, rows=64, cols=256, x=A16, y=B16, batch=1, bits=3, ws=A16,
          wsb=1 << 20):
    return lib.sqllm_dense_sparse_gemv(A16, B16, bits, rp, col, val, nnz, rows, cols, x, batch, y, ws, wsb, None)


def spmv(lib, rp=A16, col=A16, val=A16, nnz=10, rows=64, cols=256, x=A16, y=B16, batch=1, ws=A16, wsb=1 << 20):
    return lib.sqllm_spmv_add(rp, col, val, nnz, rows, cols, x, batch, y, ws, wsb, None)


def test_gemv_argument_errors(lib):
    assert gemv(lib, packed=None) == 1
    assert gemv(lib, lut=None) == 1
    assert gemv(lib, x=None) == 1
    assert gemv(lib, y=None) == 1
    assert gemv(lib, bits=1) == 2
    assert gemv(lib, bits=5) == 2
    assert gemv(lib, rows=0) == 3
    assert gemv(lib, cols=0) == 3
    assert gemv(lib, cols=300) == 3
    assert gemv(lib, batch=0) == 4
    assert gemv(lib, batch=17) == 4
    assert gemv(lib, x=MIS) == 5
    assert gemv(lib, x=P(0x200008)) == 5                 # x must be 16-byte aligned
    assert gemv(lib, y=P(0x200001)) == 5
    assert gemv(lib, packed=P(0x100008)) == 5
    assert gemv(lib, lut=P(0x100004)) == 5
    # one row tile with 8192 columns is split across workgroups: workspace needed
    assert gemv(lib, cols=8192, ws=None) == 8
    assert gemv(lib, cols=8192, wsb=16) == 8
    assert gemv(lib, cols=8192, ws=P(0x100010)) == 8


def test_sparse_argument_errors(lib):
    assert fused(lib, rp=None) == 1
    assert fused(lib, col=None) == 1
    assert fused(lib, val=None) == 1
    assert fused(lib, nnz=-1) == 3
    assert fused(lib, nnz=1 << 31) == 3
    assert fused(lib, cols=65536 + 256) == 3
    assert fused(lib, rp=P(0x100002)) == 5
    assert fused(lib, col=P(0x100001)) == 5
    assert spmv(lib, rp=None) == 1
    assert spmv(lib, batch=17) == 4
    assert spmv(lib, cols=65536 + 256) == 3
    assert spmv(lib, x=MIS) == 5
    # no outliers: nothing to do, no HIP call, CSR pointers may be NULL
    assert spmv(lib, rp=None, col=None, val=None, nnz=0) == 0


def test_noalloc_shape_errors_before_any_device_call(lib):
    """Rows, columns or batch out of range come back before the entry point looks up its scratch."""
    f = lib.sqllm_dense_sparse_gemv_noalloc
    f.argtypes = [P, P, ctypes.c_int, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, ctypes.c_int, P, P]
    assert f(A16, A16, 3, None, None, None, 0, 0, 256, B16, 1, B16, None) == 3
    assert f(A16, A16, 3, None, None, None, 0, 64, 300, B16, 1, B16, None) == 3
    assert f(A16, A16, 3, None, None, None, 0, 64, 256, B16, 17, B16, None) == 4
    assert f(A16, A16, 3, None, None, None, 0, 64, 256, B16, 0, B16, None) == 4


def test_noalloc_words_fit_the_scratch(nwpkg):
    """At the default launch shapes no accepted shape needs more than 2 MiB of
    combine words (at most about 256 row tiles are split, into two), so the
    16 MiB scratch of sqllm_dense_sparse_gemv_noalloc holds every call's words."""
    scratch = 16 << 20
    worst = 0
    for rows in [*range(1, 3000, 37), *range(3000, 70000, 997), 1 << 20, (1 << 22) + 5]:
        for cols in (256, 4096, 22016, 65536):
            for batch in (1, 4, 5, 8, 9, 16):
                for nnz in (0, 500000):
                    (p,), _ = nwpkg.launch_plan([(rows, cols, nnz)], batch=batch, workspace_bytes=scratch)
                    tiles = p["slice_tiles"] or (rows + 63) // 64
                    worst = max(worst, tiles * (p["split"] - 1) * batch * 64 * 8)
    assert 0 < worst <= 2 << 20


def test_pack_and_reader_argument_errors(lib):
    assert lib.sqllm_pack(None, 64, 256, 3, A16, B16, 256, None) == 1
    assert lib.sqllm_pack(A16, 64, 256, 3, None, B16, 256, None) == 1
    assert lib.sqllm_pack(A16, 64, 256, 3, B16, None, 256, None) == 1      # the error flag is the caller's
    assert lib.sqllm_pack(A16, 64, 256, 7, B16, B16, 256, None) == 2
    assert lib.sqllm_pack(A16, 64, 255, 3, B16, B16, 256, None) == 3
    assert lib.sqllm_pack(P(0x100001), 64, 256, 3, B16, B16, 256, None) == 5
    assert lib.sqllm_pack(A16, 64, 256, 3, B16, B16, 3, None) == 8         # flag word too small
    assert lib.sqllm_pack(A16, 64, 256, 3, B16, MIS, 256, None) == 8       # flag word misaligned
    assert lib.sqllm_test_unpack(A16, 64, 256, 3, None, None) == 1
    assert lib.sqllm_test_decode(A16, None, 64, 256, 3, B16, None) == 1
    assert lib.sqllm_test_decode(A16, B16, 64, 256, 1, B16, None) == 2


def _products(nwpkg, n, **over):
    arr = (nwpkg.Product * max(n, 1))()
    for k in range(max(n, 1)):
        f = dict(packed=A16.value, lut=B16.value, row_ptr=A16.value, col_idx=A16.value, val=A16.value, nnz=10,
                 rows=64, cols=256, x=A16.value, y=B16.value)
        f.update(over)
        arr[k] = nwpkg.Product(**f)
    return arr


def group(lib, nwpkg, n=2, bits=3, batch=1, ws=A16, wsb=1 << 20, **over):
    return lib.sqllm_dense_sparse_gemv_group(_products(nwpkg, n, **over), n, bits, batch, ws, wsb, None)


def test_group_argument_errors(lib, nwpkg):
    assert lib.sqllm_dense_sparse_gemv_group(None, 2, 3, 1, A16, 1 << 20, None) == 1
    assert group(lib, nwpkg, n=0) == 3
    assert group(lib, nwpkg, n=9) == 3
    assert group(lib, nwpkg, bits=1) == 2
    assert group(lib, nwpkg, batch=17) == 4
    assert group(lib, nwpkg, packed=None) == 1
    assert group(lib, nwpkg, x=None) == 1
    assert group(lib, nwpkg, row_ptr=None) == 1
    assert group(lib, nwpkg, cols=300) == 3
    assert group(lib, nwpkg, nnz=-1) == 3
    assert group(lib, nwpkg, x=MIS.value) == 5
    assert group(lib, nwpkg, lut=0x100004) == 5
    assert group(lib, nwpkg, ws=P(0x100010)) == 8
    # split workgroups need the workspace: one tile of 8192 columns is split
    assert group(lib, nwpkg, n=1, cols=8192, ws=None) == 8
    assert group(lib, nwpkg, n=1, cols=8192, wsb=16) == 8
    # outlier plans: helpers need the plan, 4-byte aligned, at most 8 per row tile
    assert group(lib, nwpkg, plan=None, plan_helpers=1) == 1
    assert group(lib, nwpkg, plan=0x100002, plan_helpers=1) == 5
    assert group(lib, nwpkg, plan=A16.value, plan_helpers=9) == 3      # one tile of 64 rows
    assert group(lib, nwpkg, plan=A16.value, plan_helpers=-1) == 3
    # a planned tile combines up to 16 partial sums: 15 words per output are needed
    assert group(lib, nwpkg, n=1, plan=A16.value, plan_helpers=1, wsb=15 * 64 * 8 - 1) == 8


def _plan(nwpkg, counts, rows=None):
    """Row pointers with `counts` nonzeros per row (the rest empty), and their outlier plan."""
    counts = list(counts)
    rows = rows or len(counts)
    counts += [0] * (rows - len(counts))
    rp = [0]
    for c in counts:
        rp.append(rp[-1] + c)
    return nwpkg.outlier_plan(rp)


def test_outlier_plan_rule(nwpkg):
    """A tile above twice the average tile's nonzeros gets ceil(n / q) - 1 helpers (at most 8),
    q = 2 ceil(nnz / tiles); entries (t << 4) | e follow in tile order."""
    # 4 tiles of 64 rows holding 10, 10, 10 and 370 nonzeros: q = 2 * 100 = 200, the last tile gets 1
    counts = [0] * 256
    for t, n in enumerate((10, 10, 10, 370)):
        counts[64 * t] = n
    plan = _plan(nwpkg, counts)
    assert list(plan) == [1, 0, 0, 0, 1, (3 << 4) | 0]
    # a 5000-nonzero tile among 7 of 100: q = 2 * ceil(5700 / 8) = 1426, ceil(5000 / 1426) - 1 = 3
    counts = [0] * 512
    for t in range(8):
        counts[64 * t + 5] = 100 if t != 2 else 5000
    plan = _plan(nwpkg, counts)
    assert list(plan[:9]) == [3, 0, 0, 3, 0, 0, 0, 0, 0]
    assert list(plan[9:]) == [(2 << 4) | 0, (2 << 4) | 1, (2 << 4) | 2]
    # capped at 8 helpers per tile; a ragged last tile (2 rows) counts as a tile: 100 tiles, 99 of 10
    # nonzeros and the last of 100000, q = 2 * ceil(100990 / 100) = 2020, ceil(100000 / 2020) - 1 = 49 -> 8
    counts = [0] * (64 * 99 + 2)
    for t in range(99):
        counts[64 * t] = 10
    counts[-1] = 100000
    plan = _plan(nwpkg, counts)
    assert plan[0] == 8 and not plan[1:100].any() and plan[100] == 8
    assert list(plan[101:]) == [(99 << 4) | e for e in range(8)]
    # uniform rows and an empty CSR get no helpers
    assert list(_plan(nwpkg, [3] * 1000)[:1]) == [0]
    assert list(_plan(nwpkg, [0] * 100)) == [0, 0, 0]


def test_stream_read_argument_errors(lib):
    f = lib.sqllm_test_stream_read
    assert f(None, 1024, B16, None) == 1
    assert f(A16, 1024, None, None) == 1
    assert f(A16, 0, B16, None) == 3
    assert f(A16, 1000, B16, None) == 3                 # whole KiB only
    assert f(P(0x100008), 1024, B16, None) == 5
    assert f(A16, 1024, P(0x200002), None) == 5


def test_outlier_plan_errors(lib, nwpkg):
    f = lib.sqllm_outlier_plan
    rp = (ctypes.c_int32 * 3)(0, 2, 5)
    buf = (ctypes.c_int32 * 16)()
    assert lib.sqllm_outlier_plan_len(2) == 1 + 1 + 8
    assert lib.sqllm_outlier_plan_len(0) == 0
    assert f(rp, 2, buf, 16) == 2
    assert f(None, 2, buf, 16) == 0
    assert f(rp, 2, None, 16) == 0
    assert f(rp, 2, buf, 9) == 0                      # below sqllm_outlier_plan_len
    assert f(rp, 0, buf, 16) == 0
    bad = (ctypes.c_int32 * 3)(1, 2, 5)               # must start at 0
    assert f(bad, 2, buf, 16) == 0
    bad = (ctypes.c_int32 * 3)(0, 5, 2)               # and never decrease
    assert f(bad, 2, buf, 16) == 0
    with pytest.raises(ValueError):
        nwpkg.outlier_plan([0, 3, 1])


def test_group_workspace_bytes(lib, nwpkg):
    arr = _products(nwpkg, 3, rows=100)
    assert lib.sqllm_group_workspace_bytes(arr, 3, 2) == 3 * nwpkg.workspace_bytes(100, 256, 2)
    assert lib.sqllm_group_workspace_bytes(arr, 0, 1) == 0
    assert lib.sqllm_group_workspace_bytes(arr, 3, 17) == 0
    assert lib.sqllm_group_workspace_bytes(_products(nwpkg, 2, cols=100), 2, 1) == 0


def test_tuning_hook_bounds(lib):
    assert lib.sqllm_test_tuning(0, 0, 17, 0, 0, 0) == 3      # split above 16
    assert lib.sqllm_test_tuning(0, 0, 0, 17, 0, 0) == 3      # more than 16 waves
    assert lib.sqllm_test_tuning(0, 0, 0, 0, 2, 0) == 3       # outlier form 0 or 1
    assert lib.sqllm_test_tuning(0, 0, 0, 0, 0, 2) == 3       # dense form 0 or 1
    assert lib.sqllm_test_tuning(0, 0, 0, 0, 0, 0) == 0


def test_quantize_argument_errors(lib):
    u16 = ctypes.c_uint16
    lo, hi, ts, nnz = u16(), u16(), ctypes.c_float(), ctypes.c_int64()
    ws = P(0x200000)
    wsb = lib.sqllm_quantize_workspace_bytes(64, 256)
    assert wsb == 65536 * 4 + 256 + 64 * 4
    assert lib.sqllm_quantize_workspace_bytes(64, 65537) == 0
    assert lib.sqllm_quantize_workspace_bytes(1 << 20, 4096) == 0       # more than 2^31 - 1 weights
    assert lib.sqllm_quantize_workspace_bytes(0, 256) == 0

    def thr(w=A16, sens=None, rows=64, cols=256, ppm=2000, top=500, ws=ws, wsb=wsb, out=True, t_s=True):
        refs = (ctypes.byref(lo), ctypes.byref(hi)) if out else (None, None)
        return lib.sqllm_outlier_thresholds(w, sens, rows, cols, ppm, top, ws, wsb, *refs,
                                            ctypes.byref(ts) if t_s else None, ctypes.byref(nnz), None)
    assert thr(w=None) == 1
    assert thr(out=False) == 1
    assert thr(sens=B16, t_s=False) == 1                                  # T_s needs somewhere to go
    assert thr(cols=65537) == 3
    assert thr(ppm=500000) == 3
    assert thr(ppm=-1) == 3
    assert thr(sens=B16, top=1000000) == 3
    assert thr(sens=B16, top=-1) == 3
    assert thr(w=P(0x100001)) == 5
    assert thr(sens=P(0x200002)) == 5
    assert thr(ws=None) == 8
    assert thr(ws=P(0x200080)) == 8                                      # not 256-byte aligned
    assert thr(wsb=wsb - 1) == 8

    def ext(w=A16, sens=None, rp=A16, cap=10, col=B16, dense=B16, sd=None, ws=ws, wsb=wsb):
        return lib.sqllm_outlier_extract(w, sens, 64, 256, 0x8000, 0, 1.0, rp, col, B16, cap, dense, sd, ws, wsb,
                                         None)
    assert ext(rp=None) == 1
    assert ext(dense=None) == 1
    assert ext(col=None) == 1
    assert ext(sd=B16) == 1                                               # zeroed sensitivities need sens
    assert ext(cap=-1) == 3
    assert ext(rp=P(0x100002)) == 5
    assert ext(sens=B16, sd=P(0x200002)) == 5
    assert ext(wsb=0) == 8

    def km(d=A16, bits=3, iters=10, codes=B16, lut=B16, sens=None):
        return lib.sqllm_kmeans_lut(d, sens, 64, 256, bits, iters, codes, lut, None)
    assert km(d=None) == 1
    assert km(codes=None) == 1
    assert km(bits=1) == 2
    assert km(iters=1001) == 3
    assert km(lut=P(0x100001)) == 5
    assert km(sens=P(0x100002)) == 5


def test_binding_refuses_host_tensors(nwpkg):
    import torch
    with pytest.raises(ValueError):
        nwpkg.pack(torch.zeros((64, 256), dtype=torch.uint8), 3)


LLAMA7B = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]


def test_bytes_accounting_against_table1(nwpkg):
    """Average bits per weight of LLaMA-7B's linear layers from the bytes
    formula (codes + per-row fp16 tables), against the averages the pages
    print for dense-only SqueezeLLM (summary page, §3.4 "The 3/4-bit storage
    format" and §5 Table 1: 3.02 bits / 5.29x at 3-bit, 4.05 bits / 3.95x at
    4-bit).  x and y are left out: the table counts stored weights."""
    weights = sum(r * c for r, c in LLAMA7B)
    for bits, printed_avg, printed_ratio in [(3, 3.02, 5.29), (4, 4.05, 3.95)]:
        stored = sum(nwpkg.algorithmic_bytes(r, c, bits, 0, 1) - 2 * c - 2 * r for r, c in LLAMA7B)
        avg = 8 * stored / weights
        assert int(avg * 100) / 100 == printed_avg          # the table truncates: 3.027 -> 3.02
        assert round(16 / avg, 2) == printed_ratio
    # with 0.45% outliers at 4 bytes each plus int32 row pointers the average
    # is ~3.18 bits; the pages print 3.24 (about 48 bits per outlier), a
    # difference recorded as a reading, not pinned
    nnz = [int(round(0.0045 * r * c)) for r, c in LLAMA7B]
    stored = sum(nwpkg.algorithmic_bytes(r, c, 3, n, 1) - 2 * c - 2 * r for (r, c), n in zip(LLAMA7B, nnz))
    assert 3.17 < 8 * stored / weights < 3.19


LLAMA2_13B = [(5120, 5120)] * 4 + [(13824, 5120)] * 2 + [(5120, 13824)]


def test_bytes_accounting_2bit_against_appendix_f(nwpkg):
    """Dense-only 2-bit SqueezeLLM on LLaMA2-13B's linear layers: the pages
    print 2.01 average bits (summary page, Appendix F, Table F.8) -- 2 bits of
    code plus four fp16 centroids per row."""
    weights = sum(r * c for r, c in LLAMA2_13B)
    stored = sum(nwpkg.algorithmic_bytes(r, c, 2, 0, 1) - 2 * c - 2 * r for r, c in LLAMA2_13B)
    avg = 8 * stored / weights
    assert int(avg * 100) / 100 == 2.01


# ---------------------------------------------------------------- launch planning (host logic, no device)

P65 = [(8192, 8192, 301990), (22016, 8192, 811598), (8192, 22016, 811598)]


@pytest.mark.parametrize("shape,split,gps,waves,slice_tiles", [
    ((8192, 8192, 301990), 2, 16, 8, 0),      # 128 tiles: one workgroup per unit, two groups per wave
    ((22016, 8192, 811598), 2, 16, 8, 168),   # 344 tiles: 168 at split 2 + 176 whole = 512 workgroups
    ((8192, 22016, 811598), 2, 43, 16, 0),    # 43 groups per workgroup: 16 waves
    ((4096, 4096, 75497), 2, 8, 8, 0),        # at least 8 groups per workgroup caps the split
    ((11008, 4096, 202899), 1, 16, 8, 0),     # 172 tiles: split rounded down (344 workgroups measured slower)
    ((13824, 5120, 318505), 1, 20, 12, 0),    # 20 groups per workgroup: 12 waves
    ((5120, 13824, 318505), 3, 18, 12, 0),    # 80 tiles: floor(256 / 80) = 3
    ((64, 22016, 6000), 10, 9, 8, 0),         # one tile: split up to the 8-group floor
    ((150 * 64, 4096, 1000), 2, 8, 8, 0),     # 150 tiles would leave 41% of the units idle: one split more
])
def test_single_call_launch_rules(nwpkg, shape, split, gps, waves, slice_tiles):
    (plan,), form = nwpkg.launch_plan([shape])
    assert (plan["split"], plan["gps"], plan["waves"], plan["slice_tiles"]) == (split, gps, waves, slice_tiles)
    assert form == "matrix"


def test_row_slices_need_the_workspace_words(nwpkg):
    """Without room for the first slice's words the product runs whole at split 1."""
    (plan,), _ = nwpkg.launch_plan([P65[1]], workspace_bytes=0)
    assert (plan["split"], plan["slice_tiles"]) == (1, 0)
    words = 168 * 64 * 8  # (fp32 sum, count) per row of the 168 tiles, batch 1
    (plan,), _ = nwpkg.launch_plan([P65[1]], workspace_bytes=words)
    assert plan["slice_tiles"] == 168
    (plan,), _ = nwpkg.launch_plan([P65[1]], workspace_bytes=words - 8)
    assert plan["slice_tiles"] == 0


def test_group_launch_rules(nwpkg):
    # (q, k, v): 384 tiles; q at split 2 fills one slot of every unit, k and v the other
    plans, _ = nwpkg.launch_plan([P65[0]] * 3, mode=2)
    assert [(p["split"], p["gps"], p["waves"]) for p in plans] == [(2, 16, 8), (1, 32, 8), (1, 32, 8)]
    # (gate, up): 688 tiles, whole tiles (every mix of half tiles measured slower)
    plans, _ = nwpkg.launch_plan([P65[1]] * 2, mode=2)
    assert [(p["split"], p["waves"]) for p in plans] == [(1, 8), (1, 8)]
    # (o) and (down) alone
    assert nwpkg.launch_plan([P65[0]], mode=1)[0][0]["split"] == 2
    assert [nwpkg.launch_plan([P65[2]], mode=1)[0][0][k] for k in ("split", "gps", "waves")] == [2, 43, 16]
    # products without outliers go to a launch of their own, planned from their own tiles
    plans, _ = nwpkg.launch_plan([P65[0], (8192, 8192, 0)], mode=1)
    assert [p["split"] for p in plans] == [2, 2]


def test_transposed_x_rule(nwpkg):
    """From batch 5, outliers gather from a transposed x when the products reading that x carry at least
    400K nonzeros and the workspace holds it."""
    assert nwpkg.launch_plan([P65[0]] * 3, batch=8, mode=2)[0][0]["xt"] == 1      # 906K nonzeros share one x
    assert nwpkg.launch_plan([P65[0]] * 3, batch=8, mode=1)[0][0]["xt"] == 0      # 302K each
    assert nwpkg.launch_plan([P65[0]] * 3, batch=4, mode=2)[0][0]["xt"] == 0      # below batch 5
    assert nwpkg.launch_plan([P65[1]], batch=6)[0][0]["xt"] == 1
    small = nwpkg.workspace_bytes(22016, 8192, 6) - 1
    assert nwpkg.launch_plan([P65[1]], batch=6, workspace_bytes=small)[0][0]["xt"] == 0


def test_compact_table_rule(nwpkg):
    """Fused 3-bit launches at batch 2..8 take the compact pair table exactly
    when some product's x fits in LDS beside it and not beside the full table."""
    def compact(shapes, batch, mode=0):
        return [p["compact"] for p in nwpkg.launch_plan(shapes, batch=batch, mode=mode)[0]]
    assert compact([P65[0]], 8) == [1]            # 128 KB of x: beside 32 KB, not beside 64 KB
    assert [nwpkg.launch_plan([P65[0]], batch=8)[0][0][k] for k in ("xt", "x_lds")] == [0, 1]
    assert compact([P65[0]], 1) == [0]            # batch 1: the full table only
    assert compact([P65[1]], 4) == [1]            # two workgroups per unit: 64 KB of x beside 16 KB
    assert compact([P65[1]], 8) == [0]            # fits neither way: the transposed x
    assert [nwpkg.launch_plan([P65[1]], batch=8)[0][0][k] for k in ("xt", "x_lds")] == [1, 0]
    assert compact([P65[2]], 2) == [0]            # 88 KB of x fits beside the full table
    assert compact([P65[2]], 4) == [0]            # 176 KB fits neither way
    assert [nwpkg.launch_plan([P65[2]], batch=4)[0][0][k] for k in ("xt", "x_lds")] == [0, 0]  # read in place
    assert compact([(8192, 8192, 0)], 8) == [0]   # no outliers, no staged x
    assert compact([P65[0]] * 3, 4, mode=2) == [1, 1, 1]
    assert compact([(2048, 6144, 9000)], 9) == [0]  # above batch 8 the full table, though x would fit beside a compact one
    try:
        nwpkg.set_tuning(dot_only=1)
        assert compact([P65[1]], 4) == [0]        # the dot form keeps the full table
    finally:
        nwpkg.set_tuning()


def test_dense_form_rule(nwpkg):
    try:
        nwpkg.set_tuning(dot_only=1)
        assert nwpkg.launch_plan([P65[0]], batch=8)[1] == "dot"
        assert nwpkg.launch_plan([P65[0]], batch=9)[1] == "matrix"   # no dot form above batch 8
    finally:
        nwpkg.set_tuning()
    assert nwpkg.launch_plan([P65[0]], batch=1)[1] == "matrix"


def test_forced_shapes_turn_the_rules_off(nwpkg):
    try:
        nwpkg.set_tuning(split=1)
        (plan,), _ = nwpkg.launch_plan([P65[1]])
        assert (plan["split"], plan["slice_tiles"]) == (1, 0)
        plans, _ = nwpkg.launch_plan([P65[0]] * 3, mode=2)
        assert [p["split"] for p in plans] == [1, 1, 1]
    finally:
        nwpkg.set_tuning()


def test_environment_does_not_change_a_launch(nwpkg):
    """Launch shapes come from the shapes alone: environment variables named like the knobs change nothing."""
    import subprocess
    import sys
    code = ("import json, non_uniform_weight_amd as nw; "
            "print(json.dumps([nw.launch_plan(s, batch=b) for s in ([(22016, 8192, 0)], [(8192, 8192, 30000)]) "
            "for b in (1, 6)]))")
    env = dict(os.environ, SQLLM_SPLIT="3", SQLLM_WAVES="4", SQLLM_TARGET_WGS="7", SQLLM_MIN_GPS="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True,
                         timeout=120, check=True).stdout
    import json
    want = [nwpkg.launch_plan(s, batch=b) for s in ([(22016, 8192, 0)], [(8192, 8192, 30000)]) for b in (1, 6)]
    assert json.loads(out.strip().splitlines()[-1]) == json.loads(json.dumps(want))


def test_launch_plan_argument_errors(lib):
    one = (ctypes.c_int64 * 1)(64)
    cols = (ctypes.c_int64 * 1)(256)
    nnz = (ctypes.c_int64 * 1)(0)
    out = (ctypes.c_int * 6)()
    f = lib.sqllm_test_launch_plan
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_size_t, ctypes.c_void_p]
    assert f(0, 1, one, cols, nnz, 1, 0, out) == 0
    assert f(0, 2, one, cols, nnz, 1, 0, out) != 0        # a single call plans one product
    assert f(3, 1, one, cols, nnz, 1, 0, out) != 0
    assert f(0, 1, one, cols, nnz, 17, 0, out) != 0
    assert f(0, 1, one, (ctypes.c_int64 * 1)(300), nnz, 1, 0, out) != 0   # cols not a multiple of 256
    assert f(0, 1, None, cols, nnz, 1, 0, out) != 0
