"""The benchmark's headline stream checked in full: the 80-layer
LLaMA-65B-shaped weight stream (560 products, 3-bit codes, 0.45% uniform
outliers, batch 1), run through exactly the launches the benchmark times
(four sqllm_dense_sparse_gemv_group launches per layer, captured once in a
HIP graph and replayed), and every output row of every product compared with
the oracle.  The one-call-per-product pass (sqllm_dense_sparse_gemv, also
replayed from a graph) is checked against the same oracle outputs.

The stream is built once per module (about 26 GB resident); the oracle
regenerates each matrix from its seed and runs layer range by layer range,
so that every test stays well inside the per-test time limit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev_to_u16, step

pytestmark = pytest.mark.gpu

TOL = 5e-3
SEED = 0
LAYERS = 80
CHUNK = 10  # layers per test


def _replay(ws, step_fn, stream):
    """Capture step_fn in a graph, poison every y, replay twice (with host
    work and a synchronisation between the replays) and return both
    snapshots of all outputs."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step_fn(stream)
    snaps = []
    for _ in range(2):
        for d in ws.mats:
            d["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        snaps.append([dev_to_u16(d["y"]) for d in ws.mats])
    del g
    return snaps


@pytest.fixture(scope="module")
def stream_outputs():
    import bench

    specs = synth.workload(5, bits=3, density_bp=45)
    assert len(specs) == 7 * LAYERS
    step("stream parity: building the 80-layer 3-bit 0.45% stream")
    ws = bench.WeightStream(specs, SEED)
    stream = torch.cuda.Stream()
    step(f"stream parity: graph replay of the group launches ({len(ws.groups)} launches)")
    grouped = _replay(ws, ws.step_grouped, stream)
    step(f"stream parity: graph replay of the single calls ({len(ws.calls)} calls)")
    single = _replay(ws, ws.step, stream)
    out = {"specs": specs, "grouped": grouped, "single": single}
    del ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def test_replays_are_bit_identical(stream_outputs):
    for name in ("grouped", "single"):
        a, b = stream_outputs[name]
        bad = [i for i in range(len(a)) if not np.array_equal(a[i], b[i])]
        assert not bad, f"{name}: replays differ in products {bad[:10]}"


@pytest.mark.parametrize("chunk", range(LAYERS // CHUNK))
def test_every_row_matches_oracle(stream_outputs, chunk):
    specs = stream_outputs["specs"]
    lo, hi = 7 * CHUNK * chunk, 7 * CHUNK * (chunk + 1)
    step(f"stream parity: oracle over products {lo}..{hi - 1}")
    worst = {"grouped": 0.0, "single": 0.0}
    for i in range(lo, hi):
        spec = specs[i]
        m = synth.make_matrix(spec, seed=SEED, workload=5, index=i)
        assert m.col.size == spec.nnz
        y_ref, scale = oracle.dense_sparse_gemv(m.codes, m.lut, spec.bits, m.row_ptr, m.col, m.val, m.x)
        for name in ("grouped", "single"):
            y = stream_outputs[name][1][i]
            assert y.shape == (1, spec.rows)
            ok, err = oracle.within_tolerance(y, y_ref, scale, TOL)
            assert ok, f"{name} product {i} ({spec.name}): max normalised error {err:.3e} > {TOL}"
            worst[name] = max(worst[name], err)
    print(f"products {lo}..{hi - 1}: worst normalised error {worst}")
