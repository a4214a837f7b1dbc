"""sqllm_dense_sparse_gemv_noalloc: the fused product with the library's
fixed per-GPU scratch in place of a workspace equals sqllm_dense_sparse_gemv
bit for bit (same launch, same summation order), on consecutive calls of
decreasing size that share the scratch, and refuses a launch whose words
exceed the scratch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DevMatrix, dev_to_u16, nw, step
from seeds import stable_seed

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _noalloc(d: DevMatrix) -> torch.Tensor:
    y = torch.full((d.x.shape[0], d.rows), float("nan"), dtype=torch.float16, device="cuda")
    return nw().dense_sparse_gemv_noalloc(d.packed, d.lut, d.bits, d.row_ptr, d.col, d.val, d.x, y)


def _with_workspace(d: DevMatrix) -> torch.Tensor:
    ws = torch.zeros(nw().workspace_bytes(d.rows, d.cols, d.x.shape[0]), dtype=torch.uint8, device="cuda")
    return d.fused(ws=ws)


# (rows, cols, bits, batch, outlier density in basis points): the first call
# splits its 128 row tiles in two and gathers from the transposed x (811K
# outliers at batch 6); the second, smaller one splits 16 tiles eight ways at
# batch 1; the third, smaller still, has no outliers and splits 5 tiles four
# ways; the fourth stages x (128 KB at batch 8) beside the compact 3-bit pair
# table.
CASES = [(8192, 22016, 3, 6, 45), (1024, 16384, 4, 1, 45), (300, 8192, 3, 2, 0), (300, 8192, 3, 8, 45)]


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    mats = []
    for i, (rows, cols, bits, batch, bp) in enumerate(CASES):
        spec = synth.MatrixSpec(f"noalloc{i}", rows, cols, bits, batch, bp)
        mats.append((spec, synth.make_matrix(spec, seed=0, workload=9, index=i)))
    plans = [nw().launch_plan([(s.rows, s.cols, s.nnz)], batch=s.batch)[0][0] for s, _ in mats]
    assert plans[0]["split"] == 2 and plans[0]["xt"] == 1 and plans[1]["split"] == 8 and plans[2]["split"] == 4
    assert plans[3]["compact"] == 1 and plans[3]["x_lds"] == 1
    for (spec, m), plan in zip(mats, plans):
        step(f"noalloc {spec.rows}x{spec.cols} bits {spec.bits} batch {spec.batch} nnz {spec.nnz} plan {plan}")
        d = DevMatrix.from_synth(m)
        y_na = dev_to_u16(_noalloc(d))
        y_ws = dev_to_u16(_with_workspace(d))
        assert np.array_equal(y_na, y_ws), f"{spec.name}: {int((y_na != y_ws).sum())} outputs differ"
        sel = np.sort(np.random.default_rng(stable_seed("noalloc", spec.rows)).choice(spec.rows, 256, replace=False))
        y_ref, scale = oracle.dense_sparse_gemv(m.codes[sel], m.lut, spec.bits, m.row_ptr, m.col, m.val, m.x,
                                                rows=spec.rows, sel=sel)
        ok, worst = oracle.within_tolerance(y_na[:, sel], y_ref, scale, TOL)
        assert ok, f"{spec.name}: max normalised error {worst:.3e}"


def test_noalloc_refuses_words_beyond_the_scratch():
    """A launch forced to 16 column splits on 22016 rows at batch 16 needs
    344 * 15 * 16 * 512 bytes of words (42 MB): refused before any launch,
    and the next call is unaffected."""
    spec = synth.MatrixSpec("noalloc_big", 22016, 8192, 3, 16, 0)
    m = synth.make_matrix(spec, seed=0, workload=9, index=7)
    d = DevMatrix.from_synth(m)
    y = torch.zeros((16, spec.rows), dtype=torch.float16, device="cuda")
    try:
        nw().set_tuning(split=16)
        step("noalloc forced split 16 (expect SQLLM_ERR_SCRATCH)")
        with pytest.raises(nw().SqllmError) as err:
            nw().dense_sparse_gemv_noalloc(d.packed, d.lut, d.bits, None, None, None, d.x, y)
        assert err.value.status == 10
    finally:
        nw().set_tuning()
    torch.cuda.synchronize()
    assert int(y.view(torch.int16).abs().sum().item()) == 0      # nothing was launched
    step("noalloc after the refusal")
    assert np.array_equal(dev_to_u16(_noalloc(d)), dev_to_u16(_with_workspace(d)))
