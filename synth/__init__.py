"""Seeded synthetic inputs for the dense-and-sparse LUT GEMV y = (D + S) x.

Thin numpy wrapper over ``libsynth.so`` (built from ``synth.c``).  The module
draws inputs only -- codes, per-row fp16 lookup tables, CSR outliers and fp16
activations -- and holds none of the product's arithmetic, so the HIP path and
the CPU oracle can both be fed from it.

The workload list mirrors the layer shapes on which SqueezeLLM is evaluated
(SqueezeLLM: Dense-and-Sparse Quantization, summary page, §5 "Experiments":
LLaMA-7B/13B/65B linear layers; §3.4 "The Dense-and-Sparse Decomposition":
0.45% = 0.05% sensitive + 0.4% outlier weights kept in fp16 CSR; Appendix C,
Figure C.1: per-channel outlier counts are heavily skewed).  The weights are
synthetic, not trained: no checkpoint or dataset is read.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# tensor kinds, folded into the stream id of every drawn tensor
KIND_CODES, KIND_LUT, KIND_X, KIND_POS, KIND_VAL, KIND_PERM = 1, 2, 3, 4, 5, 6

LUT_SIGMA = 0.02      # centroids ~ N(0, 0.02)
OUTLIER_SIGMA = 0.2   # outliers ~ N(0, 0.2): ~10x the dense spread (Figure 5 reading)
X_SIGMA = 1.0         # activations ~ N(0, 1)
ZIPF_S = 1.2


def build() -> str:
    """Compile libsynth.so with gcc (OpenMP for the bulk code draws)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_normal.restype = dbl
        L.synth_normal.argtypes = [u64, u64]
        L.synth_f16.restype = ctypes.c_uint16
        L.synth_f16.argtypes = [dbl]
        L.synth_codes.restype = None
        L.synth_codes.argtypes = [u64, i64, i64, i64, i32, vp]
        L.synth_normal_f16.restype = None
        L.synth_normal_f16.argtypes = [u64, i64, i64, dbl, vp]
        L.synth_lut.restype = None
        L.synth_lut.argtypes = [u64, i64, i64, i32, dbl, i32, vp]
        L.synth_nnz_bp.restype = i64
        L.synth_nnz_bp.argtypes = [i64, i64, i64]
        L.synth_csr_uniform.restype = i32
        L.synth_csr_uniform.argtypes = [u64, u64, i64, i64, i64, dbl, vp, vp, vp]
        L.synth_csr_zipf.restype = i32
        L.synth_csr_zipf.argtypes = [u64, u64, u64, i64, i64, i64, dbl, dbl, vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, stream: int) -> int:
    return int(lib().synth_key(seed & (2**64 - 1), stream & (2**64 - 1)))


def stream_id(kind: int, workload: int, matrix: int) -> int:
    return (kind << 48) | (workload << 40) | matrix


def f16_bits(v: float) -> int:
    return int(lib().synth_f16(float(v)))


def codes(k: int, rows: int, cols: int, bits: int, row0: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """uint8 [rows, cols] codes of rows row0 .. row0+rows-1, uniform in [0, 2^bits)."""
    assert cols % 8 == 0
    if out is None:
        out = np.empty((rows, cols), dtype=np.uint8)
    lib().synth_codes(k, row0, rows, cols, bits, _ptr(out))
    return out


def normal_f16(k: int, n: int, sigma: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_f16(k, start, n, sigma, _ptr(out))
    return out


def lut(k: int, rows: int, bits: int, sigma: float = LUT_SIGMA, sorted_: bool = True, row0: int = 0) -> np.ndarray:
    """uint16 (fp16 bits) [rows, 2^bits]."""
    out = np.empty((rows, 1 << bits), dtype=np.uint16)
    lib().synth_lut(k, row0, rows, bits, sigma, 1 if sorted_ else 0, _ptr(out))
    return out


def nnz_bp(rows: int, cols: int, bp: int) -> int:
    return int(lib().synth_nnz_bp(rows, cols, bp))


def csr_uniform(k_pos: int, k_val: int, rows: int, cols: int, nnz: int, sigma: float = OUTLIER_SIGMA):
    row_ptr = np.empty(rows + 1, dtype=np.int32)
    col = np.empty(max(nnz, 1), dtype=np.uint16)
    val = np.empty(max(nnz, 1), dtype=np.uint16)
    rc = lib().synth_csr_uniform(k_pos, k_val, rows, cols, nnz, sigma, _ptr(row_ptr), _ptr(col), _ptr(val))
    if rc != 0:
        raise ValueError("synth_csr_uniform: bad arguments")
    return row_ptr, col[:nnz], val[:nnz]


def csr_zipf(k_perm: int, k_pos: int, k_val: int, rows: int, cols: int, nnz: int, s: float = ZIPF_S,
             sigma: float = OUTLIER_SIGMA):
    row_ptr = np.empty(rows + 1, dtype=np.int32)
    col = np.empty(max(nnz, 1), dtype=np.uint16)
    val = np.empty(max(nnz, 1), dtype=np.uint16)
    rc = lib().synth_csr_zipf(k_perm, k_pos, k_val, rows, cols, nnz, s, sigma, _ptr(row_ptr), _ptr(col), _ptr(val))
    if rc != 0:
        raise ValueError("synth_csr_zipf: bad arguments")
    return row_ptr, col[:nnz], val[:nnz]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class MatrixSpec:
    """One linear layer y = (D + S) x: rows = out features, cols = in features."""
    name: str
    rows: int
    cols: int
    bits: int
    batch: int = 1
    density_bp: int = 45          # outlier density in basis points (45 = 0.45%)
    zipf: bool = False            # skewed per-row outlier counts

    @property
    def nnz(self) -> int:
        return nnz_bp(self.rows, self.cols, self.density_bp)


@dataclass
class Matrix:
    spec: MatrixSpec
    codes: np.ndarray      # uint8 [rows, cols]
    lut: np.ndarray        # uint16 [rows, 2^bits]
    row_ptr: np.ndarray    # int32 [rows + 1]
    col: np.ndarray        # uint16 [nnz]
    val: np.ndarray        # uint16 [nnz]
    x: np.ndarray          # uint16 [batch, cols]
    keys: dict = field(default_factory=dict)


def matrix_keys(seed: int, workload: int, index: int) -> dict:
    return {kind: key(seed, stream_id(kind, workload, index))
            for kind in (KIND_CODES, KIND_LUT, KIND_X, KIND_POS, KIND_VAL, KIND_PERM)}


def make_sparse(spec: MatrixSpec, keys: dict):
    nnz = spec.nnz
    if spec.zipf:
        return csr_zipf(keys[KIND_PERM], keys[KIND_POS], keys[KIND_VAL], spec.rows, spec.cols, nnz)
    return csr_uniform(keys[KIND_POS], keys[KIND_VAL], spec.rows, spec.cols, nnz)


def make_matrix(spec: MatrixSpec, seed: int = 0, workload: int = 0, index: int = 0,
                with_codes: bool = True) -> Matrix:
    ks = matrix_keys(seed, workload, index)
    c = codes(ks[KIND_CODES], spec.rows, spec.cols, spec.bits) if with_codes else None
    lt = lut(ks[KIND_LUT], spec.rows, spec.bits)
    rp, ci, cv = make_sparse(spec, ks)
    x = normal_f16(ks[KIND_X], spec.batch * spec.cols, X_SIGMA).reshape(spec.batch, spec.cols)
    return Matrix(spec, c, lt, rp, ci, cv, x, ks)


def codes_rows(m: Matrix, row_list) -> np.ndarray:
    """Regenerate the codes of selected rows only (uint8 [len(row_list), cols])."""
    out = np.empty((len(row_list), m.spec.cols), dtype=np.uint8)
    for i, r in enumerate(row_list):
        codes(m.keys[KIND_CODES], 1, m.spec.cols, m.spec.bits, row0=int(r), out=out[i:i + 1])
    return out


LLAMA65B_LINEARS = (("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
                    ("gate", 22016, 8192), ("up", 22016, 8192), ("down", 8192, 22016))
LLAMA13B_LINEARS = (("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
                    ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824))


def workload(n: int, bits: int | None = None, density_bp: int | None = None, batch: int | None = None):
    """Matrix specs of the five evaluation workloads (1-based, as listed):

    1. one LLaMA-7B q_proj 4096x4096, 3-bit, 0.45% uniform outliers, batch 1;
    2. LLaMA-7B MLP pair up 11008x4096 + down 4096x11008, 4-bit, 0.45%, batch 1;
    3. one LLaMA-13B decoder layer (7 linears), 3-bit, 0.45% Zipf(1.2) rows;
    4. LLaMA-65B shapes 8192x8192, 22016x8192, 8192x22016, 3-bit, 0.45%, batch 1/2/4/8;
    5. the 80-layer LLaMA-65B stream (560 linears), 3/4-bit, 0 / 0.05 / 0.45%.
    """
    if n == 1:
        return [MatrixSpec("q_proj", 4096, 4096, 3)]
    if n == 2:
        return [MatrixSpec("up", 11008, 4096, 4), MatrixSpec("down", 4096, 11008, 4)]
    if n == 3:
        return [MatrixSpec(nm, r, c, 3, zipf=True) for nm, r, c in LLAMA13B_LINEARS]
    if n == 4:
        b = batch or 1
        return [MatrixSpec("q", 8192, 8192, 3, b), MatrixSpec("gate", 22016, 8192, 3, b),
                MatrixSpec("down", 8192, 22016, 3, b)]
    if n == 5:
        bt = 3 if bits is None else bits
        d = 45 if density_bp is None else density_bp
        return [MatrixSpec(f"L{layer}.{nm}", r, c, bt, 1, d)
                for layer in range(80) for nm, r, c in LLAMA65B_LINEARS]
    raise ValueError(n)
