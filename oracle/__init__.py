"""CPU oracle for the dense-and-sparse LUT GEMV y = (D + S) x (fp64).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The product path
(``non_uniform_weight_amd``) never imports it, and it never imports the
product path.  The arithmetic lives in ``sqllm_oracle.c`` (plain C); this
file only marshals numpy arrays through ctypes.

Which passages each function follows is stated beside each C function:
SqueezeLLM: Dense-and-Sparse Quantization (summary page), §3.2 "Big-Picture
Architecture", §3.4 "The Dense-and-Sparse Decomposition", "Kernel
Implementation" and "The 3/4-bit storage format".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (plain C99, OpenMP over rows)."""
    src = os.path.join(_HERE, "sqllm_oracle.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_f16.argtypes = [dbl]
        L.oracle_packed_bytes.restype = i64
        L.oracle_packed_bytes.argtypes = [i64, i64, i32]
        L.oracle_unpack.restype = None
        L.oracle_unpack.argtypes = [vp, i64, i64, i32, vp]
        L.oracle_decode.restype = None
        L.oracle_decode.argtypes = [vp, vp, i64, i64, i32, vp]
        L.oracle_dense_sparse_gemv.restype = i32
        L.oracle_dense_sparse_gemv.argtypes = [vp, vp, i32, vp, vp, vp, i64, i64, vp, i64, vp, i32, vp, vp, i32]
        L.oracle_spmv_add.restype = i32
        L.oracle_spmv_add.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp, i32, vp, vp, vp, i32]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "contiguous numpy array expected"
    return a.ctypes.data


def f16_to_f64(h: int) -> float:
    return float(lib().oracle_f16_to_f64(int(h)))


def f64_to_f16(v: float) -> int:
    return int(lib().oracle_f64_to_f16(float(v)))


_F16_TABLE = None


def f16_array_to_f64(h: np.ndarray) -> np.ndarray:
    """Decode fp16 bit patterns with the oracle's decoder (tabulated once over
    all 65536 patterns)."""
    global _F16_TABLE
    if _F16_TABLE is None:
        f = lib().oracle_f16_to_f64
        _F16_TABLE = np.fromiter((f(i) for i in range(65536)), dtype=np.float64, count=65536)
    return _F16_TABLE[np.asarray(h, dtype=np.uint16)]


def f64_array_to_f16(v: np.ndarray) -> np.ndarray:
    f = lib().oracle_f64_to_f16
    flat = np.ascontiguousarray(v, dtype=np.float64).ravel()
    return np.fromiter((f(float(t)) for t in flat), dtype=np.uint16, count=flat.size).reshape(v.shape)


def packed_bytes(rows: int, cols: int, bits: int) -> int:
    return int(lib().oracle_packed_bytes(rows, cols, bits))


def unpack(packed: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size >= packed_bytes(rows, cols, bits)
    out = np.empty((rows, cols), dtype=np.uint8)
    lib().oracle_unpack(_p(packed), rows, cols, bits, _p(out))
    return out


def decode(codes: np.ndarray, lut: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    lut = np.ascontiguousarray(lut, dtype=np.uint16)
    rows, cols = codes.shape
    out = np.empty((rows, cols), dtype=np.uint16)
    lib().oracle_decode(_p(codes), _p(lut), rows, cols, bits, _p(out))
    return out


def dense_sparse_gemv(codes, lut, bits, row_ptr, col, val, x, rows=None, sel=None, threads=0):
    """fp64 y, scale [batch][nsel].  codes: uint8 [nsel][cols] (rows in sel order);
    row_ptr None -> dense part only."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    lut = np.ascontiguousarray(lut, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    batch, cols = x.shape
    rows = lut.shape[0] if rows is None else rows
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        nsel = sel.size
    else:
        nsel = rows
    assert codes.shape == (nsel, cols)
    if row_ptr is not None:
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        col = np.ascontiguousarray(col, dtype=np.uint16)
        val = np.ascontiguousarray(val, dtype=np.uint16)
        if col.size == 0:
            col = np.zeros(1, np.uint16)
            val = np.zeros(1, np.uint16)
    y = np.empty((batch, nsel), dtype=np.float64)
    s = np.empty((batch, nsel), dtype=np.float64)
    rc = lib().oracle_dense_sparse_gemv(_p(codes), _p(lut), bits, _p(row_ptr), _p(col), _p(val), rows, cols,
                                        _p(sel), nsel, _p(x), batch, _p(y), _p(s), threads)
    if rc != 0:
        raise ValueError("oracle_dense_sparse_gemv: bad arguments")
    return y, s


def spmv_add(row_ptr, col, val, x, y_in, rows, sel=None, threads=0):
    """fp64 y = y_in + S x and its normaliser, [batch][nsel]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    batch, cols = x.shape
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.uint16)
    val = np.ascontiguousarray(val, dtype=np.uint16)
    if col.size == 0:
        col = np.zeros(1, np.uint16)
        val = np.zeros(1, np.uint16)
    y_in = np.ascontiguousarray(y_in, dtype=np.uint16).reshape(batch, rows)
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        nsel = sel.size
    else:
        nsel = rows
    y = np.empty((batch, nsel), dtype=np.float64)
    s = np.empty((batch, nsel), dtype=np.float64)
    rc = lib().oracle_spmv_add(_p(row_ptr), _p(col), _p(val), rows, cols, _p(sel), nsel, _p(x), batch, _p(y_in),
                               _p(y), _p(s), threads)
    if rc != 0:
        raise ValueError("oracle_spmv_add: bad arguments")
    return y, s


def within_tolerance(y_dev_f16: np.ndarray, y_ref: np.ndarray, scale: np.ndarray, tol: float = 5e-3):
    """Acceptance rule: |y_dev - y_ref| <= tol * scale per output; scale == 0
    requires y_dev == 0.  Returns (ok, max normalised error)."""
    yd = f16_array_to_f64(y_dev_f16) if y_dev_f16.dtype == np.uint16 else np.asarray(y_dev_f16, np.float64)
    err = np.abs(yd - y_ref)
    zero = scale == 0
    ok_zero = np.all(yd[zero] == 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(zero, 0.0, err / np.where(zero, 1.0, scale))
    worst = float(norm.max()) if norm.size else 0.0
    return bool(ok_zero and worst <= tol), worst
