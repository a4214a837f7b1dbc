"""Helpers shared by the GPU parity tests: move generator output to the
device through the C ABI (pack on the GPU) and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth


def nw():
    import non_uniform_weight_amd
    return non_uniform_weight_amd


def step(msg: str) -> None:
    """Name the case before a GPU step, so a crash can be traced to it."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def u16_to_dev(a: np.ndarray, dtype=torch.float16) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    return t.view(dtype) if dtype != torch.int16 else t


def dev_to_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class DevMatrix:
    """Device copies of one generated layer (codes packed by sqllm_pack)."""

    def __init__(self, codes, lut, bits, row_ptr, col, val, x):
        self.rows, self.cols = lut.shape[0], x.shape[-1]
        self.bits = bits
        self.packed = nw().pack(torch.from_numpy(np.ascontiguousarray(codes)).cuda(), bits)
        self.lut = u16_to_dev(lut)
        self.nnz = int(col.size) if col is not None else 0
        if self.nnz:
            self.row_ptr = torch.from_numpy(np.ascontiguousarray(row_ptr, dtype=np.int32)).cuda()
            self.col = u16_to_dev(col, torch.int16)
            self.val = u16_to_dev(val)
        else:
            self.row_ptr = self.col = self.val = None
        self.x = u16_to_dev(np.ascontiguousarray(x).reshape(-1, self.cols))

    @classmethod
    def from_synth(cls, m: synth.Matrix):
        return cls(m.codes, m.lut, m.spec.bits, m.row_ptr, m.col, m.val, m.x)

    def fused(self, y=None, ws=None):
        return nw().dense_sparse_gemv(self.packed, self.lut, self.bits, self.row_ptr, self.col, self.val, self.x,
                                      y=y, ws=ws)

    def gemv(self, y=None, ws=None):
        return nw().gemv(self.packed, self.lut, self.bits, self.x, y=y, ws=ws)

    def spmv_add(self, y, ws=None):
        if self.nnz == 0:
            rp = torch.zeros(self.rows + 1, dtype=torch.int32, device="cuda")
            return nw().spmv_add(rp, None, None, self.x, y, ws=ws)
        return nw().spmv_add(self.row_ptr, self.col, self.val, self.x, y, ws=ws)


def assert_close(y_dev: torch.Tensor, y_ref: np.ndarray, scale: np.ndarray, tol: float = 5e-3, what: str = ""):
    yd = dev_to_u16(y_dev)
    ok, worst = oracle.within_tolerance(yd, y_ref, scale, tol)
    assert ok, f"{what}: max normalised error {worst:.3e} > {tol} (or nonzero where the normaliser is 0)"
    return worst


def reference(codes, lut, bits, row_ptr, col, val, x, sel=None):
    rows = lut.shape[0]
    if sel is None:
        return oracle.dense_sparse_gemv(codes, lut, bits, row_ptr, col, val, x, rows=rows)
    return oracle.dense_sparse_gemv(codes[sel] if codes.shape[0] == rows else codes, lut, bits, row_ptr, col, val,
                                    x, rows=rows, sel=np.asarray(sel))
