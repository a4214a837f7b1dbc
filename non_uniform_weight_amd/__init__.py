"""MI355X (gfx950) dense-and-sparse LUT matrix-vector product y = (D + S) x.

Thin ctypes binding over ``libsqllm.so`` (see ``include/sqllm.h``): it checks
tensor dtypes, shapes and devices, passes raw device pointers and the current
HIP stream, and turns status codes into exceptions.  Every step of the
product runs in the library's HIP kernels; there is no fallback path.  If the
library has not been built (``__graft_entry__.build()`` or
``python non_uniform_weight_amd/_build.py``) importing this package raises.

The operation follows SqueezeLLM: Dense-and-Sparse Quantization (summary
page), §3.4 "The Dense-and-Sparse Decomposition" (W = D + S, S in CSR) and
"Kernel Implementation" (LUT-based dense kernel, balanced sparse kernel,
fused into one launch).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loads the HIP runtime first, so libsqllm.so binds to the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsqllm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python non_uniform_weight_amd/_build.py)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_lib.sqllm_status_string.restype = ctypes.c_char_p
_lib.sqllm_status_string.argtypes = [_i32]
_lib.sqllm_packed_bytes.restype = _sz
_lib.sqllm_packed_bytes.argtypes = [_i64, _i64, _i32]
_lib.sqllm_workspace_bytes.restype = _sz
_lib.sqllm_workspace_bytes.argtypes = [_i64, _i64, _i32]
_lib.sqllm_pack.restype = _i32
_lib.sqllm_pack.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _sz, _vp]
_lib.sqllm_gemv.restype = _i32
_lib.sqllm_gemv.argtypes = [_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]
_lib.sqllm_spmv_add.restype = _i32
_lib.sqllm_spmv_add.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]
_lib.sqllm_dense_sparse_gemv.restype = _i32
_lib.sqllm_dense_sparse_gemv.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                         _sz, _vp]
_lib.sqllm_dense_sparse_gemv_noalloc.restype = _i32
_lib.sqllm_dense_sparse_gemv_noalloc.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp,
                                                 _vp]


class Product(ctypes.Structure):
    """One item of sqllm_dense_sparse_gemv_group (sqllm_product)."""
    _fields_ = [("packed", _vp), ("lut", _vp), ("row_ptr", _vp), ("col_idx", _vp), ("val", _vp), ("nnz", _i64),
                ("rows", _i64), ("cols", _i64), ("x", _vp), ("y", _vp), ("plan", _vp), ("plan_helpers", _i64)]


_lib.sqllm_outlier_plan_len.restype = _sz
_lib.sqllm_outlier_plan_len.argtypes = [_i64]
_lib.sqllm_outlier_plan.restype = _sz
_lib.sqllm_outlier_plan.argtypes = [_vp, _i64, _vp, _sz]
_lib.sqllm_group_workspace_bytes.restype = _sz
_lib.sqllm_group_workspace_bytes.argtypes = [ctypes.POINTER(Product), _i32, _i32]
_lib.sqllm_dense_sparse_gemv_group.restype = _i32
_lib.sqllm_dense_sparse_gemv_group.argtypes = [ctypes.POINTER(Product), _i32, _i32, _i32, _vp, _sz, _vp]
_lib.sqllm_quantize_workspace_bytes.restype = _sz
_lib.sqllm_quantize_workspace_bytes.argtypes = [_i64, _i64]
_lib.sqllm_outlier_thresholds.restype = _i32
_lib.sqllm_outlier_thresholds.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _vp, _sz, ctypes.POINTER(ctypes.c_uint16),
                                          ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(_i64), _vp]
_lib.sqllm_outlier_extract.restype = _i32
_lib.sqllm_outlier_extract.argtypes = [_vp, _vp, _i64, _i64, ctypes.c_uint16, ctypes.c_uint16, ctypes.c_float, _vp,
                                       _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]
_lib.sqllm_kmeans_lut.restype = _i32
_lib.sqllm_kmeans_lut.argtypes = [_vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp]
_lib.sqllm_test_unpack.restype = _i32
_lib.sqllm_test_unpack.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp]
_lib.sqllm_test_tuning.restype = _i32
_lib.sqllm_test_tuning.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
_lib.sqllm_test_launch_plan.restype = _i32
_lib.sqllm_test_launch_plan.argtypes = [_i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                        _i32, _sz, ctypes.POINTER(_i32)]
_lib.sqllm_test_stream_read.restype = _i32
_lib.sqllm_test_stream_read.argtypes = [_vp, _sz, _vp, _vp]
_lib.sqllm_test_decode.restype = _i32
_lib.sqllm_test_decode.argtypes = [_vp, _vp, _i64, _i64, _i32, _vp, _vp]

EXPORTS = ("sqllm_status_string", "sqllm_packed_bytes", "sqllm_workspace_bytes", "sqllm_pack", "sqllm_gemv",
           "sqllm_spmv_add", "sqllm_dense_sparse_gemv", "sqllm_group_workspace_bytes",
           "sqllm_dense_sparse_gemv_group", "sqllm_quantize_workspace_bytes", "sqllm_outlier_thresholds",
           "sqllm_outlier_extract", "sqllm_kmeans_lut", "sqllm_test_unpack", "sqllm_test_decode", "sqllm_test_tuning",
           "sqllm_test_launch_plan", "sqllm_dense_sparse_gemv_noalloc", "sqllm_outlier_plan_len",
           "sqllm_outlier_plan", "sqllm_test_stream_read")
MAX_GROUP = 8

SQLLM_OK = 0


class SqllmError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_lib.sqllm_status_string(status).decode()}")


def _check(status: int, call: str) -> None:
    if status != SQLLM_OK:
        raise SqllmError(status, call)


def library() -> ctypes.CDLL:
    return _lib


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: torch.Tensor expected")
    if not t.is_cuda:
        raise ValueError(f"{name}: device tensor expected (the product runs only on the GPU)")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {dtype} expected, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: contiguous tensor expected")
    return t.data_ptr()


def packed_bytes(rows: int, cols: int, bits: int) -> int:
    return int(_lib.sqllm_packed_bytes(rows, cols, bits))


def workspace_bytes(rows: int, cols: int, batch: int) -> int:
    return int(_lib.sqllm_workspace_bytes(rows, cols, batch))


_WORKSPACES: dict = {}


def workspace(rows: int, cols: int, batch: int, device=None, stream=None) -> torch.Tensor:
    """Zero-filled workspace cached per (device, stream), grown on demand.
    The calls leave it all zero again; calls on one stream are ordered, so
    they may share it, and each stream gets its own."""
    return _cached_workspace(workspace_bytes(rows, cols, batch), device, stream)


def _cached_workspace(nbytes: int, device=None, stream=None) -> torch.Tensor:
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.index, s.cuda_stream)
    need = max(nbytes, 256)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        # zeroed on the stream that will use it, so the fill is ordered before
        # the call; a smaller buffer it replaces is freed to that same stream
        with torch.cuda.stream(s):
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """uint8 codes [rows, cols] -> packed uint8 buffer (synchronises the stream)."""
    rows, cols = codes.shape
    n = packed_bytes(rows, cols, bits)
    if n == 0:
        raise ValueError(f"pack: unsupported shape/bits ({rows}, {cols}, {bits})")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    if out.numel() < n:
        raise ValueError("pack: output buffer too small")
    cp, op = _dev(codes, "codes", torch.uint8), _dev(out, "packed", torch.uint8)
    flag = _cached_workspace(256, codes.device, stream)  # the call's error flag; the call leaves it zero
    _check(_lib.sqllm_pack(cp, rows, cols, bits, op, flag.data_ptr(), flag.numel(), _stream(stream)), "sqllm_pack")
    return out


def _x_y(x: torch.Tensor, y: torch.Tensor | None, rows: int):
    if x.dim() == 1:
        x = x.unsqueeze(0)
    batch, cols = x.shape
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float16, device=x.device)
    if tuple(y.shape) != (batch, rows):
        raise ValueError(f"y: shape {(batch, rows)} expected, got {tuple(y.shape)}")
    return x, y, batch, cols


def gemv(packed, lut, bits, x, y=None, ws=None, stream=None) -> torch.Tensor:
    """y = D x (dense part)."""
    rows = lut.shape[0]
    x, y, batch, cols = _x_y(x, y, rows)
    ws = workspace(rows, cols, batch, x.device, stream) if ws is None else ws
    _check(_lib.sqllm_gemv(_dev(packed, "packed", torch.uint8), _dev(lut, "lut", torch.float16), bits, rows, cols,
                           _dev(x, "x", torch.float16), batch, _dev(y, "y", torch.float16),
                           _dev(ws, "workspace", torch.uint8), ws.numel(), _stream(stream)), "sqllm_gemv")
    return y


def _csr_ptrs(row_ptr, col, val):
    nnz = int(col.numel()) if col is not None else 0
    if nnz == 0:
        return None, None, None, 0
    col_dtype = torch.uint16 if col.dtype == torch.uint16 else torch.int16  # 16-bit column bits
    return (_dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col_idx", col_dtype),
            _dev(val, "val", torch.float16), nnz)


def spmv_add(row_ptr, col, val, x, y, ws=None, stream=None) -> torch.Tensor:
    """y += S x in place (col: uint16, or int16 holding the same bits)."""
    rows = row_ptr.shape[0] - 1
    x, y, batch, cols = _x_y(x, y, rows)
    ws = workspace(rows, cols, batch, x.device, stream) if ws is None else ws
    rp, ci, cv, nnz = _csr_ptrs(row_ptr, col, val)
    _check(_lib.sqllm_spmv_add(rp, ci, cv, nnz, rows, cols, _dev(x, "x", torch.float16), batch,
                               _dev(y, "y", torch.float16), _dev(ws, "workspace", torch.uint8), ws.numel(),
                               _stream(stream)), "sqllm_spmv_add")
    return y


def dense_sparse_gemv(packed, lut, bits, row_ptr, col, val, x, y=None, ws=None, stream=None) -> torch.Tensor:
    """y = (D + S) x in one launch."""
    rows = lut.shape[0]
    x, y, batch, cols = _x_y(x, y, rows)
    ws = workspace(rows, cols, batch, x.device, stream) if ws is None else ws
    rp, ci, cv, nnz = _csr_ptrs(row_ptr, col, val)
    _check(_lib.sqllm_dense_sparse_gemv(_dev(packed, "packed", torch.uint8), _dev(lut, "lut", torch.float16), bits,
                                        rp, ci, cv, nnz, rows, cols, _dev(x, "x", torch.float16), batch,
                                        _dev(y, "y", torch.float16), _dev(ws, "workspace", torch.uint8), ws.numel(),
                                        _stream(stream)), "sqllm_dense_sparse_gemv")
    return y


def dense_sparse_gemv_noalloc(packed, lut, bits, row_ptr, col, val, x, y, stream=None) -> torch.Tensor:
    """y = (D + S) x with the library's fixed per-GPU scratch instead of a
    workspace; y must be given (nothing is allocated on this path)."""
    rows = lut.shape[0]
    if y is None:
        raise ValueError("dense_sparse_gemv_noalloc: y must be given")
    x, y, batch, cols = _x_y(x, y, rows)
    rp, ci, cv, nnz = _csr_ptrs(row_ptr, col, val)
    _check(_lib.sqllm_dense_sparse_gemv_noalloc(_dev(packed, "packed", torch.uint8), _dev(lut, "lut", torch.float16),
                                                bits, rp, ci, cv, nnz, rows, cols, _dev(x, "x", torch.float16), batch,
                                                _dev(y, "y", torch.float16), _stream(stream)),
           "sqllm_dense_sparse_gemv_noalloc")
    return y


def outlier_plan(row_ptr) -> np.ndarray:
    """Offline: the outlier plan of a CSR (sqllm_outlier_plan) from its row
    pointers (host array or tensor, int32 [rows + 1]); int32 entries, the
    helper count first.  Copy it to the device for a group item's "plan"."""
    rp = np.ascontiguousarray(row_ptr.cpu().numpy() if isinstance(row_ptr, torch.Tensor) else row_ptr,
                              dtype=np.int32)
    rows = rp.size - 1
    cap = int(_lib.sqllm_outlier_plan_len(rows))
    if cap == 0:
        raise ValueError(f"outlier_plan: unsupported row count {rows}")
    out = np.zeros(cap, dtype=np.int32)
    n = int(_lib.sqllm_outlier_plan(rp.ctypes.data, rows, out.ctypes.data, cap))
    if n == 0:
        raise ValueError("outlier_plan: row pointers must start at 0 and never decrease")
    return out[:n]


def group_products(items, bits: int):
    """ctypes array of sqllm_product from dicts with keys packed, lut, row_ptr,
    col, val, x, y (tensors; row_ptr/col/val may be None) and optionally plan
    (device int32 tensor from outlier_plan)."""
    arr = (Product * len(items))()
    batch = None
    for k, it in enumerate(items):
        rows = it["lut"].shape[0]
        x, y, b, cols = _x_y(it["x"], it["y"], rows)
        if batch is not None and b != batch:
            raise ValueError("group: every product must have the same batch")
        batch = b
        rp, ci, cv, nnz = _csr_ptrs(it.get("row_ptr"), it.get("col"), it.get("val"))
        plan = it.get("plan")
        pp, ph = None, 0
        if plan is not None:
            pp = _dev(plan, "plan", torch.int32)
            ph = int(it["plan_helpers"]) if "plan_helpers" in it else int(plan[0].item())  # the latter syncs
        arr[k] = Product(_dev(it["packed"], "packed", torch.uint8), _dev(it["lut"], "lut", torch.float16), rp, ci, cv,
                         nnz, rows, cols, _dev(x, "x", torch.float16), _dev(y, "y", torch.float16), pp, ph)
    return arr, batch


def stream_read(src: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None, stream=None) -> None:
    """Test-only: read nbytes (default all) of src once; sink (int32 [4096] on the device) receives each
    wave's XOR of the 32-bit words it read."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if not (src.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 4096):
        raise ValueError("stream_read: device src and an int32 device sink of 4096 entries expected")
    _check(_lib.sqllm_test_stream_read(src.data_ptr(), n, sink.data_ptr(), _stream(stream)), "sqllm_test_stream_read")


def group_workspace_bytes(items, bits: int) -> int:
    arr, batch = group_products(items, bits)
    return int(_lib.sqllm_group_workspace_bytes(arr, len(items), batch))


def dense_sparse_gemv_group(items, bits: int, ws: torch.Tensor | None = None, stream=None) -> None:
    """y_i = (D_i + S_i) x_i for up to 8 independent products in one launch.
    items: dicts with packed, lut, row_ptr, col, val, x and y (y preallocated
    fp16 [batch, rows]); ws: zero-filled uint8 workspace of at least
    group_workspace_bytes(items, bits) bytes (a cached one if None)."""
    arr, batch = group_products(items, bits)
    need = int(_lib.sqllm_group_workspace_bytes(arr, len(items), batch))
    if ws is None:
        ws = _cached_workspace(need, items[0]["x"].device, stream)
    _check(_lib.sqllm_dense_sparse_gemv_group(arr, len(items), bits, batch, _dev(ws, "workspace", torch.uint8),
                                              ws.numel(), _stream(stream)), "sqllm_dense_sparse_gemv_group")


def _quantize_ws(rows: int, cols: int, device) -> torch.Tensor:
    n = int(_lib.sqllm_quantize_workspace_bytes(rows, cols))
    if n == 0:
        raise ValueError(f"unsupported shape ({rows}, {cols})")
    return torch.empty(n, dtype=torch.uint8, device=device)


def outlier_thresholds(w: torch.Tensor, tail_ppm: int = 2000, sens: torch.Tensor | None = None, top_ppm: int = 0,
                       stream=None):
    """(T_min, T_max, T_s, nnz) of an fp16 [rows, cols] weight matrix: fp16
    bit patterns as ints, T_s a float (+inf without sensitivities); synchronises."""
    rows, cols = w.shape
    ws = _quantize_ws(rows, cols, w.device)
    lo, hi, ts, nnz = ctypes.c_uint16(), ctypes.c_uint16(), ctypes.c_float(), ctypes.c_int64()
    sp = None if sens is None else _dev(sens, "sens", torch.float32)
    _check(_lib.sqllm_outlier_thresholds(_dev(w, "w", torch.float16), sp, rows, cols, tail_ppm, top_ppm,
                                         ws.data_ptr(), ws.numel(), ctypes.byref(lo), ctypes.byref(hi),
                                         ctypes.byref(ts), ctypes.byref(nnz), _stream(stream)),
           "sqllm_outlier_thresholds")
    return lo.value, hi.value, ts.value, nnz.value


def outlier_extract(w: torch.Tensor, t_min: int, t_max: int, nnz: int, sens: torch.Tensor | None = None,
                    t_s: float = float("inf"), stream=None):
    """W = D + S: (row_ptr int32, col int16 bits, val fp16, dense fp16, and,
    given sens, the sensitivities with zeros at S's entries); synchronises."""
    rows, cols = w.shape
    ws = _quantize_ws(rows, cols, w.device)
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=w.device)
    col = torch.empty(max(nnz, 1), dtype=torch.int16, device=w.device)
    val = torch.empty(max(nnz, 1), dtype=torch.float16, device=w.device)
    dense = torch.empty_like(w)
    sp = sd = None
    sens_dense = None
    if sens is not None:
        sp = _dev(sens, "sens", torch.float32)
        sens_dense = torch.empty_like(sens)
        sd = sens_dense.data_ptr()
    _check(_lib.sqllm_outlier_extract(_dev(w, "w", torch.float16), sp, rows, cols, t_min, t_max, t_s,
                                      row_ptr.data_ptr(), col.data_ptr(), val.data_ptr(), nnz,
                                      _dev(dense, "dense", torch.float16), sd, ws.data_ptr(), ws.numel(),
                                      _stream(stream)), "sqllm_outlier_extract")
    if sens is None:
        return row_ptr, col[:nnz], val[:nnz], dense
    return row_ptr, col[:nnz], val[:nnz], dense, sens_dense


def kmeans_lut(dense: torch.Tensor, bits: int, iters: int = 20, sens: torch.Tensor | None = None, stream=None):
    """Per-row k-means codes (uint8 [rows, cols]) and fp16 tables [rows, 2^bits] of D."""
    rows, cols = dense.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=dense.device)
    lut = torch.empty((rows, 1 << bits), dtype=torch.float16, device=dense.device)
    sp = None if sens is None else _dev(sens, "sens", torch.float32)
    _check(_lib.sqllm_kmeans_lut(_dev(dense, "dense", torch.float16), sp, rows, cols, bits, iters,
                                 _dev(codes, "codes", torch.uint8), _dev(lut, "lut", torch.float16), _stream(stream)),
           "sqllm_kmeans_lut")
    return codes, lut


def unpack_codes(packed, rows, cols, bits, stream=None) -> torch.Tensor:
    """Test-only reader: packed -> uint8 codes [rows, cols] (sqllm_test_unpack)."""
    out = torch.empty((rows, cols), dtype=torch.uint8, device=packed.device)
    _check(_lib.sqllm_test_unpack(_dev(packed, "packed", torch.uint8), rows, cols, bits, _dev(out, "codes", torch.uint8),
                                  _stream(stream)), "sqllm_test_unpack")
    return out


def decode_weights(packed, lut, rows, cols, bits, stream=None) -> torch.Tensor:
    """Test-only reader: fp16 LUT[r][code[r][c]] [rows, cols] (sqllm_test_decode)."""
    out = torch.empty((rows, cols), dtype=torch.float16, device=packed.device)
    _check(_lib.sqllm_test_decode(_dev(packed, "packed", torch.uint8), _dev(lut, "lut", torch.float16), rows, cols,
                                  bits, _dev(out, "w", torch.float16), _stream(stream)), "sqllm_test_decode")
    return out


def set_tuning(target_wgs: int = 0, min_gps: int = 0, split: int = 0, waves: int = 0,
               sparse_naive: int = 0, dot_only: int = 0) -> None:
    """Test-only: launch shape of later calls (0 = default); sparse_naive=1 selects the unbalanced
    one-thread-per-row outlier form, dot_only=1 the v_dot2c dense form instead of the matrix cores
    (ablations)."""
    _check(_lib.sqllm_test_tuning(target_wgs, min_gps, split, waves, sparse_naive, dot_only),
           "sqllm_test_tuning")


def launch_plan(shapes, batch: int = 1, workspace_bytes: int = 1 << 30, mode: int = 0):
    """Test-only: the launch the calls would make for products of (rows, cols, nnz) in `shapes`, without a
    device.  mode 0: one sqllm_dense_sparse_gemv; 1: one group call, a separate x per product; 2: one
    group call, one shared x.  Per product: dict(split, gps, waves, xt, x_lds, slice_tiles, compact); plus the
    form.  xt: the outliers read a transposed copy of x; x_lds: they read x staged in LDS; compact: the launch
    takes the compact 3-bit pair table (which leaves room in LDS for x)."""
    n = len(shapes)
    arr = lambda k: (_i64 * n)(*[int(sh[k]) for sh in shapes])
    out = (_i32 * (5 * n + 1))()
    _check(_lib.sqllm_test_launch_plan(mode, n, arr(0), arr(1), arr(2), batch, workspace_bytes, out),
           "sqllm_test_launch_plan")
    items = [dict(split=out[5 * i], gps=out[5 * i + 1], waves=out[5 * i + 2], xt=int(out[5 * i + 3] == 1),
                  x_lds=int(out[5 * i + 3] == 2), slice_tiles=out[5 * i + 4], compact=int(bool(out[5 * n] & 2)))
             for i in range(n)]
    return items, ("matrix" if out[5 * n] & 1 else "dot")


def algorithmic_bytes(rows: int, cols: int, bits: int, nnz: int, batch: int) -> int:
    """Bytes the product must move once: codes (exactly b bits each), the
    per-row fp16 tables, the CSR outliers (fp16 value + 16-bit column per
    nonzero, int32 row pointers), x and y."""
    b = rows * cols * bits // 8 + rows * (1 << bits) * 2 + 2 * batch * cols + 2 * batch * rows
    if nnz > 0:
        b += 4 * nnz + 4 * (rows + 1)
    return b
