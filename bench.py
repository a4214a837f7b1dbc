#!/usr/bin/env python3
"""Throughput of the fused dense-and-sparse LUT GEMV y = (D + S) x on one MI355X.

One step = one pass over the whole weight stream of an 80-layer
LLaMA-65B-shaped model at batch 1: 80 x (q, k, v, o 8192x8192; gate, up
22016x8192; down 8192x22016) = 560 fused products, 3-bit codes with per-row
8-entry fp16 tables and 0.45% fp16 CSR outliers, each with its own fp16
activation vector, back to back on one stream.  A decoder layer can compute
q, k and v together (one input) and gate and up together (one input), so the
default launch order is four launches of sqllm_dense_sparse_gemv_group per
layer: (q, k, v), (o), (gate, up), (down); `--launch single` makes one
sqllm_dense_sparse_gemv call per product instead.  Inputs are seeded
synthetic data of those shapes and distributions (no trained weights), all
resident in HBM before the timed region (24.3 GB of codes + 1.2 GB of CSR).

Metric: effective HBM GB/s = algorithmic bytes per step (codes at exactly b
bits + fp16 tables + CSR at 4 B per nonzero + int32 row pointers + x + y)
divided by the time per step; also microseconds per GEMV.  The pages' kernel
ran on other hardware and prints no GB/s figure, so vs_baseline is null.

Prints one JSON line.  ``--gpus`` above 1 is refused: the benchmark runs on
one GPU (sharding by output rows is described in the design notes).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--bits", type=int, default=3, choices=(2, 3, 4))
    p.add_argument("--density-bp", type=int, default=45, help="outlier density in basis points (45 = 0.45%%)")
    p.add_argument("--layers", type=int, default=80)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-graph", action="store_true", help="time plain launches only")
    p.add_argument("--launch", choices=("level", "single"), default="level",
                   help="level: one group launch per (q,k,v), (o), (gate,up), (down); single: one call per product")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-single", action="store_true",
                   help="skip the one-call-per-product pass, so that a profiler sees only the group launches")
    p.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: min(16, cpus))")
    p.add_argument("--no-per-matrix", action="store_true",
                   help="skip the cold single-matrix timings of the 7B, 7B-MLP, 13B and 65B shapes at batch 1 and the "
                        "launch-structure ceiling (the stream's launches as plain reads)")
    p.add_argument("--ablation", choices=("outliers", "batch", "offline", "configs", "ceiling"), default=None,
                   help="outliers: time each product of the 13B (skewed rows) and 65B (uniform) workloads "
                        "dense-only, with balanced outliers, with one-thread-per-row outliers, and stream-ordered "
                        "(one JSON line of its own); batch: the 65B shapes at batch 1, 2, 4, 8, 16 in both dense forms; offline: the "
                        "dense-and-sparse split and weighted k-means of one 65B layer, with the oracle on a sample; configs: "
                        "every matrix of the 7B, 7B-MLP, 13B and 65B single-matrix workloads, cold and warm; ceiling: the "
                        "stream's launches as plain reads of the same bytes with no arithmetic")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="after the timing, copy BYTES device-to-device once (a reference for counter runs)")
    return p.parse_args()


class WeightStream:
    """Device-resident weight stream; launches go through the C ABI with
    arguments marshalled once."""

    def __init__(self, specs, seed: int, workload_id: int = 5, progress_every: int = 70):
        import numpy as np
        import torch

        import non_uniform_weight_amd as nw
        import synth

        self.nw, self.torch, self.np = nw, torch, np
        self.specs = specs
        self.bits = specs[0].bits
        self.mats = []
        self.bytes_per_step = 0
        rows_max = max(s.rows for s in specs)
        cols_max = max(s.cols for s in specs)
        batch = max(s.batch for s in specs)
        # a group launch gives every product its own slots: room for three
        self.ws = torch.zeros(max(3 * nw.workspace_bytes(rows_max, cols_max, batch), 256), dtype=torch.uint8,
                              device="cuda")
        t0 = time.time()
        for i, spec in enumerate(specs):
            m = synth.make_matrix(spec, seed=seed, workload=workload_id, index=i)
            codes = torch.from_numpy(m.codes).cuda()
            packed = nw.pack(codes, spec.bits)
            del codes
            d = {
                "spec": spec,
                "packed": packed,
                "lut": torch.from_numpy(m.lut.view(np.int16)).cuda().view(torch.float16),
                "row_ptr": torch.from_numpy(m.row_ptr).cuda(),
                "col": torch.from_numpy(m.col.view(np.int16)).cuda() if m.col.size else None,
                "val": torch.from_numpy(m.val.view(np.int16)).cuda().view(torch.float16) if m.col.size else None,
                "x": torch.from_numpy(m.x.view(np.int16)).cuda().view(torch.float16),
                "y": torch.empty((spec.batch, spec.rows), dtype=torch.float16, device="cuda"),
                "nnz": int(m.col.size),
            }
            d["bytes"] = nw.algorithmic_bytes(spec.rows, spec.cols, spec.bits, d["nnz"], spec.batch)
            self.bytes_per_step += d["bytes"]
            self.mats.append(d)
            if (i + 1) % progress_every == 0 or i + 1 == len(specs):
                log(f"resident: {i + 1}/{len(specs)} matrices, {self.bytes_per_step / 1e9:.2f} GB, "
                    f"{time.time() - t0:.0f} s")
        torch.cuda.synchronize()
        self._marshal()

    LEVELS = ((0, 1, 2), (3,), (4, 5), (6,))  # per layer: (q, k, v), (o), (gate, up), (down)

    def _marshal(self):
        lib = self.nw.library()
        self.fn = lib.sqllm_dense_sparse_gemv
        self.group_fn = lib.sqllm_dense_sparse_gemv_group
        vp = ctypes.c_void_p
        self.groups = []
        for l0 in range(0, len(self.mats), 7):
            for lv in self.LEVELS:
                ids = [l0 + i for i in lv if l0 + i < len(self.mats)]
                if not ids:
                    continue
                arr = (self.nw.Product * len(ids))()
                for k, i in enumerate(ids):
                    d = self.mats[i]
                    sp, nnz = d["spec"], d["nnz"]
                    arr[k] = self.nw.Product(d["packed"].data_ptr(), d["lut"].data_ptr(),
                                             d["row_ptr"].data_ptr() if nnz else None,
                                             d["col"].data_ptr() if nnz else None,
                                             d["val"].data_ptr() if nnz else None, nnz, sp.rows, sp.cols,
                                             d["x"].data_ptr(), d["y"].data_ptr())
                need = int(lib.sqllm_group_workspace_bytes(arr, len(ids), self.specs[ids[0]].batch))
                assert 0 < need <= self.ws.numel(), (need, self.ws.numel())
                self.groups.append((arr, len(ids), self.specs[ids[0]].batch))
        self.calls = []
        for d in self.mats:
            s = d["spec"]
            nnz = d["nnz"]
            self.calls.append((
                vp(d["packed"].data_ptr()), vp(d["lut"].data_ptr()), s.bits,
                vp(d["row_ptr"].data_ptr()) if nnz else None,
                vp(d["col"].data_ptr()) if nnz else None,
                vp(d["val"].data_ptr()) if nnz else None,
                nnz, s.rows, s.cols, vp(d["x"].data_ptr()), s.batch, vp(d["y"].data_ptr()),
                vp(self.ws.data_ptr()), self.ws.numel()))

    def step(self, stream) -> None:
        fn, h = self.fn, vp_stream(stream)
        for args in self.calls:
            st = fn(*args, h)
            if st != 0:
                raise RuntimeError(f"sqllm_dense_sparse_gemv failed with status {st}")

    def step_grouped(self, stream) -> None:
        fn, h = self.group_fn, vp_stream(stream)
        ws, wsb = ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel()
        for arr, n, batch in self.groups:
            st = fn(arr, n, self.bits, batch, ws, wsb, h)
            if st != 0:
                raise RuntimeError(f"sqllm_dense_sparse_gemv_group failed with status {st}")


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    if it was taken on the kernel sources as they are now (else None)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "non_uniform_weight_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    sha = h.hexdigest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md")):
        fields = {}
        with open(path) as fh:
            for line in fh:
                if " = " in line:
                    k, v = line.rsplit(" = ", 1)
                    fields[k.strip().split()[-1]] = v.strip()
        if (fields.get("kernel_sources_sha256") == sha and fields.get("roofline_kernel") == kernel
                and "traffic_bytes_per_launch" in fields):
            return int(float(fields["traffic_bytes_per_launch"]))
    return None


def copy_calibration(nbytes: int) -> None:
    """One plain device-to-device copy of nbytes (read nbytes, write nbytes):
    the reference that scales hardware byte counters in profiling runs."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes")


def vp_stream(stream):
    return ctypes.c_void_p(stream.cuda_stream)


def cpu_baseline(stream_specs, seed: int, threads: int, min_seconds: float = 10.0):
    """The oracle as it stands, on layer 0 (7 linears, every row), passes
    repeated until it has run for min_seconds (at most 20 passes)."""
    import oracle
    import synth

    import non_uniform_weight_amd as nw

    mats = [synth.make_matrix(spec, seed=seed, workload=5, index=i) for i, spec in enumerate(stream_specs[:7])]
    total_bytes = 0
    elapsed = 0.0
    passes = 0
    while passes < 20 and (passes == 0 or elapsed < min_seconds):
        for m in mats:
            spec = m.spec
            t0 = time.perf_counter()
            oracle.dense_sparse_gemv(m.codes, m.lut, spec.bits, m.row_ptr if m.col.size else None, m.col, m.val,
                                     m.x, threads=threads)
            elapsed += time.perf_counter() - t0
            total_bytes += nw.algorithmic_bytes(spec.rows, spec.cols, spec.bits, int(m.col.size), spec.batch)
        passes += 1
    # the same oracle on one thread, over the layer's first linear once (a few seconds)
    m = mats[0]
    t0 = time.perf_counter()
    oracle.dense_sparse_gemv(m.codes, m.lut, m.spec.bits, m.row_ptr if m.col.size else None, m.col, m.val, m.x,
                             threads=1)
    t1 = time.perf_counter() - t0
    b1 = nw.algorithmic_bytes(m.spec.rows, m.spec.cols, m.spec.bits, int(m.col.size), m.spec.batch)
    return {"value": round(total_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of the stream: 7 linears, all rows, {passes} passes ({total_bytes / 1e6:.1f} MB "
                      f"algorithmic), fp64 oracle incl. the |W||x| normaliser, {elapsed:.1f} s",
            "cpu_model": _cpu_model(), "cpus_visible": os.cpu_count(),
            "single_thread": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"{m.spec.rows}x{m.spec.cols} once, {t1:.1f} s"}}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def outlier_ablation(args) -> None:
    """Outlier cost over the dense-only product (summary page, Appendix C,
    Table C.1 measures the same for its kernels): per product of the 13B
    layer (Zipf-skewed rows) and the three 65B shapes (uniform rows), batch 1,
    graph-timed launches cycling over copies of the inputs (>= 1.2 GB, so
    nothing stays cached)."""
    import numpy as np
    import torch

    import non_uniform_weight_amd as nw
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    modes = ("dense_only", "balanced", "balanced_group", "balanced_planned", "one_thread_per_row", "stream_ordered")
    rows_out = []
    for wl, specs in ((3, synth.workload(3)), (4, synth.workload(4, batch=1))):
        for i, spec in enumerate(specs):
            m = synth.make_matrix(spec, seed=args.seed, workload=wl, index=i)
            packed = nw.pack(torch.from_numpy(m.codes).cuda(), spec.bits)
            reps = max(1, -(-1200 * 2 ** 20 // packed.numel()))
            copies = []
            for r in range(reps):
                copies.append(dict(
                    packed=packed if r == 0 else packed.clone(),
                    lut=torch.from_numpy(m.lut.view(np.int16)).cuda().view(torch.float16),
                    row_ptr=torch.from_numpy(m.row_ptr).cuda(), col=torch.from_numpy(m.col.view(np.int16)).cuda(),
                    val=torch.from_numpy(m.val.view(np.int16)).cuda().view(torch.float16)))
            x = torch.from_numpy(m.x.view(np.int16)).cuda().view(torch.float16)
            y = torch.empty((1, spec.rows), dtype=torch.float16, device="cuda")
            ws = torch.zeros(max(nw.workspace_bytes(spec.rows, spec.cols, 1), 256), dtype=torch.uint8,
                             device="cuda")
            plan_host = nw.outlier_plan(m.row_ptr)
            plan = torch.from_numpy(plan_host).cuda()
            res = {"workload": wl, "product": spec.name, "shape": f"{spec.rows}x{spec.cols}", "nnz": int(m.col.size),
                   "plan_helpers": int(plan_host[0])}
            for mode in modes:
                def call(c):
                    if mode == "dense_only":
                        nw.gemv(c["packed"], c["lut"], spec.bits, x, y=y, ws=ws, stream=stream)
                    elif mode == "stream_ordered":
                        nw.gemv(c["packed"], c["lut"], spec.bits, x, y=y, ws=ws, stream=stream)
                        nw.spmv_add(c["row_ptr"], c["col"], c["val"], x, y, ws=ws, stream=stream)
                    elif mode == "balanced_group":  # a group of one product, without the plan
                        nw.dense_sparse_gemv_group([dict(c, x=x, y=y)], spec.bits, ws=ws, stream=stream)
                    elif mode == "balanced_planned":  # the same with the outlier plan
                        nw.dense_sparse_gemv_group([dict(c, x=x, y=y, plan=plan, plan_helpers=int(plan_host[0]))],
                                                   spec.bits, ws=ws, stream=stream)
                    else:
                        nw.dense_sparse_gemv(c["packed"], c["lut"], spec.bits, c["row_ptr"], c["col"], c["val"], x,
                                             y=y, ws=ws, stream=stream)
                nw.set_tuning(sparse_naive=1 if mode == "one_thread_per_row" else 0)
                try:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        for k in range(20):
                            call(copies[k % reps])
                    with torch.cuda.stream(stream):
                        for _ in range(5):
                            g.replay()
                        torch.cuda.synchronize()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        for _ in range(10):
                            g.replay()
                        e1.record(stream)
                        torch.cuda.synchronize()
                finally:
                    nw.set_tuning()
                res[mode + "_us"] = round(e0.elapsed_time(e1) / 200 * 1e3, 3)
            for mode in modes[1:]:
                res[mode + "_overhead_pct"] = round(100 * (res[mode + "_us"] / res["dense_only_us"] - 1), 1)
            log(f"ablation {res}")
            rows_out.append(res)
            del copies, packed
            torch.cuda.empty_cache()
    summary = {}
    for wl in (3, 4):
        sel = [r for r in rows_out if r["workload"] == wl]
        base = sum(r["dense_only_us"] for r in sel)
        summary[f"workload{wl}"] = {mode: round(100 * (sum(r[mode + "_us"] for r in sel) / base - 1), 1)
                                    for mode in modes[1:]}
    print(json.dumps({"ablation": "outliers", "unit": "us per product, overhead % over dense-only",
                      "batch": 1, "products": rows_out, "overhead_pct_total": summary}), flush=True)


def batch_ablation(args) -> None:
    """The three 65B shapes (3-bit, 0.45% outliers) at batch 1, 2, 4, 8 and
    16, in both dense forms (matrix-core, the default, and v_dot2c, which is
    built up to batch 8):
    µs per product and effective GB/s (bytes grow only by x and y, the math by
    the batch), graph-timed over copies of the inputs (>= 1.2 GB)."""
    import numpy as np
    import torch

    import non_uniform_weight_amd as nw
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    out = []
    for batch, form in [(b, f) for b in (1, 2, 4, 8, 16) for f in ("matrix", "dot") if b <= 8 or f == "matrix"]:
        nw.set_tuning(dot_only=1 if form == "dot" else 0)
        for i, spec in enumerate(synth.workload(4, batch=batch)):
            m = synth.make_matrix(spec, seed=args.seed, workload=4, index=i)
            packed = nw.pack(torch.from_numpy(m.codes).cuda(), spec.bits)
            lut = torch.from_numpy(m.lut.view(np.int16)).cuda().view(torch.float16)
            rp = torch.from_numpy(m.row_ptr).cuda()
            col = torch.from_numpy(m.col.view(np.int16)).cuda()
            val = torch.from_numpy(m.val.view(np.int16)).cuda().view(torch.float16)
            x = torch.from_numpy(m.x.view(np.int16)).cuda().view(torch.float16)
            reps = max(1, -(-1200 * 2 ** 20 // packed.numel()))
            # every copy holds its own codes, tables and CSR: nothing but x stays cache-resident
            copies = [(packed, lut, rp, col, val)] + [tuple(t.clone() for t in (packed, lut, rp, col, val))
                                                      for _ in range(reps - 1)]
            y = torch.empty((batch, spec.rows), dtype=torch.float16, device="cuda")
            ws = torch.zeros(max(nw.workspace_bytes(spec.rows, spec.cols, batch), 256), dtype=torch.uint8,
                             device="cuda")
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for k in range(20):
                    c = copies[k % reps]
                    nw.dense_sparse_gemv(c[0], c[1], spec.bits, c[2], c[3], c[4], x, y=y, ws=ws, stream=stream)
            with torch.cuda.stream(stream):
                for _ in range(5):
                    g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(10):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 200 * 1e3
            nbytes = nw.algorithmic_bytes(spec.rows, spec.cols, spec.bits, int(m.col.size), batch)
            res = {"batch": batch, "form": form, "shape": f"{spec.rows}x{spec.cols}", "us": round(us, 3),
                   "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1)}
            log(f"batch ablation {res}")
            out.append(res)
            del copies, packed, lut, rp, col, val
            torch.cuda.empty_cache()
    nw.set_tuning()
    print(json.dumps({"ablation": "batch", "unit": "us per product and effective GB/s", "products": out}),
          flush=True)


def single_matrix_timing(spec, wl: int, index: int, seed: int, stream, calls_per_trial: int = 200,
                         trials: int = 5, full: bool = False, planned: bool = False) -> dict:
    """One matrix of a single-matrix workload, one fused sqllm_dense_sparse_gemv
    per product.  Cold: every call reads its own copy of codes, tables and CSR
    (copies >= 1 GB, beyond the caches), calls_per_trial calls captured in a
    HIP graph, median of `trials` replays.  full: also a plain launch loop
    (arguments marshalled once, one C-ABI call per product) and warm (every
    call on one copy).  planned: each call is a group call of this one
    product with its outlier plan (sqllm_outlier_plan) instead."""
    import statistics

    import numpy as np
    import torch

    import non_uniform_weight_amd as nw
    import synth

    h = vp_stream(stream)
    fn = nw.library().sqllm_dense_sparse_gemv
    vp = ctypes.c_void_p
    m = synth.make_matrix(spec, seed=seed, workload=wl, index=index)
    packed = nw.pack(torch.from_numpy(m.codes).cuda(), spec.bits)
    lut = torch.from_numpy(m.lut.view(np.int16)).cuda().view(torch.float16)
    rp = torch.from_numpy(m.row_ptr).cuda()
    col = torch.from_numpy(m.col.view(np.int16)).cuda()
    val = torch.from_numpy(m.val.view(np.int16)).cuda().view(torch.float16)
    x = torch.from_numpy(m.x.view(np.int16)).cuda().view(torch.float16)
    y = torch.empty((spec.batch, spec.rows), dtype=torch.float16, device="cuda")
    ws = torch.zeros(max(nw.workspace_bytes(spec.rows, spec.cols, spec.batch), 256), dtype=torch.uint8,
                     device="cuda")
    nnz = int(m.col.size)
    plan_host = nw.outlier_plan(m.row_ptr) if planned else None
    del m
    nbytes = nw.algorithmic_bytes(spec.rows, spec.cols, spec.bits, nnz, spec.batch)
    reps = max(1, -(-1024 * 2 ** 20 // nbytes))
    copies = [(packed, lut, rp, col, val)] + [tuple(t.clone() for t in (packed, lut, rp, col, val))
                                              for _ in range(reps - 1)]
    argv = [(vp(c[0].data_ptr()), vp(c[1].data_ptr()), spec.bits, vp(c[2].data_ptr()), vp(c[3].data_ptr()),
             vp(c[4].data_ptr()), nnz, spec.rows, spec.cols, vp(x.data_ptr()), spec.batch, vp(y.data_ptr()),
             vp(ws.data_ptr()), ws.numel()) for c in copies]
    if planned:
        plan = torch.from_numpy(plan_host).cuda()
        gfn = nw.library().sqllm_dense_sparse_gemv_group
        garr = []
        for c in copies:
            arr = (nw.Product * 1)()
            arr[0] = nw.Product(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr(), c[3].data_ptr(), c[4].data_ptr(),
                                nnz, spec.rows, spec.cols, x.data_ptr(), y.data_ptr(), plan.data_ptr(),
                                int(plan_host[0]))
            garr.append(arr)

    def run(k, cold=True):
        i = k % reps if cold else 0
        if planned:
            st = gfn(garr[i], 1, spec.bits, spec.batch, vp(ws.data_ptr()), ws.numel(), h)
        else:
            st = fn(*argv[i], h)
        if st != 0:
            raise RuntimeError(f"sqllm_dense_sparse_gemv{'_group' if planned else ''} failed with status {st}")

    def graph_us(cold):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for k in range(calls_per_trial):
                run(k, cold)
        ts = []
        with torch.cuda.stream(stream):
            g.replay()  # warm-up
            torch.cuda.synchronize()
            for _ in range(trials):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / calls_per_trial)
        del g
        return statistics.median(ts)

    def plain_us():
        ts = []
        with torch.cuda.stream(stream):
            for k in range(20):
                run(k)
            torch.cuda.synchronize()
            for _ in range(trials):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for k in range(calls_per_trial):
                    run(k)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / calls_per_trial)
        return statistics.median(ts)

    cold = graph_us(True)
    ideal = nbytes / (HBM_PEAK_GBS * 1e3)
    res = {"workload": wl, "product": spec.name, "shape": f"{spec.rows}x{spec.cols}", "bits": spec.bits,
           "batch": spec.batch, "nnz": nnz, "bytes": nbytes, "copies": reps,
           "ideal_us": round(ideal, 3), "target70_us": round(ideal / 0.7, 3),
           "graph_us": round(cold, 3), "GB_per_s": round(nbytes / (cold * 1e3), 1),
           "pct_peak": round(100 * ideal / cold, 1)}
    if planned:
        res["plan_helpers"] = int(plan_host[0])
    if full:
        plain, warm = plain_us(), graph_us(False)
        res.update({"plain_us": round(plain, 3), "warm_us": round(warm, 3),
                    "warm_GB_per_s": round(nbytes / (warm * 1e3), 1)})
    del copies, argv, packed, lut, rp, col, val, x, y, ws
    if planned:
        del garr, plan
    torch.cuda.empty_cache()
    return res


def per_matrix(seed: int, stream) -> dict:
    """The single-matrix workloads, cold (copies >= 1 GB), one fused call per
    product in a HIP graph: LLaMA-7B q_proj 4096x4096 3-bit, the 7B MLP pair
    up 11008x4096 + down 4096x11008 4-bit, the LLaMA-13B layer's seven
    linears 3-bit with Zipf rows, all at batch 1, and the LLaMA-65B shapes
    8192x8192, 22016x8192, 8192x22016 3-bit at batch 1, 2, 4 and 8; all with
    0.45% outliers.  Keys of batches above 1 end in _b<batch>."""
    import synth

    names = {1: "llama7b", 2: "llama7b_mlp", 3: "llama13b", 4: "llama65b"}
    out = {}
    runs = [(wl, 1) for wl in (1, 2, 3, 4)] + [(4, b) for b in (2, 4, 8)]
    for wl, batch in runs:
        for i, spec in enumerate(synth.workload(wl, batch=batch) if wl == 4 else synth.workload(wl)):
            r = single_matrix_timing(spec, wl, i, seed, stream)
            key = f"{names[wl]}_{spec.name}_{spec.rows}x{spec.cols}_{spec.bits}bit" + (f"_b{batch}" if batch > 1 else "")
            out[key] = {"us_per_gemv": r["graph_us"], "GB_per_s": r["GB_per_s"],
                        "frac": round(r["GB_per_s"] / HBM_PEAK_GBS, 4), "nnz": r["nnz"], "copies": r["copies"]}
            log(f"per matrix {key}: {r['graph_us']:.2f} us, {r['GB_per_s']:.0f} GB/s")
            if wl == 3:  # the skewed rows, with the outlier plan (a group call of one product)
                r = single_matrix_timing(spec, wl, i, seed, stream, planned=True)
                out[key + "_planned"] = {"us_per_gemv": r["graph_us"], "GB_per_s": r["GB_per_s"],
                                         "frac": round(r["GB_per_s"] / HBM_PEAK_GBS, 4), "nnz": r["nnz"],
                                         "copies": r["copies"], "plan_helpers": r["plan_helpers"]}
                log(f"per matrix {key}_planned: {r['graph_us']:.2f} us, {r['GB_per_s']:.0f} GB/s, "
                    f"{r['plan_helpers']} helpers")
    return out


def config_table(args) -> None:
    """Each matrix of the four single-matrix workloads, one fused call per
    product: the 7B q_proj 4096x4096 (3-bit), the 7B MLP pair up 11008x4096 +
    down 4096x11008 (4-bit), the 13B layer's seven linears (3-bit, Zipf rows)
    and the three 65B shapes at batch 1, 2, 4 and 8 (3-bit), all with 0.45%
    outliers.  Cold: every call reads its own copy of codes, tables and CSR
    (copies >= 1 GB, beyond the caches), 200 calls per trial, median of 5
    trials, as a HIP graph and as a plain launch loop (arguments marshalled
    once, one C-ABI call per product).  Warm: 200 graph calls on one copy
    (cache-resident for the smaller shapes, reported apart)."""
    import statistics

    import numpy as np
    import torch

    import non_uniform_weight_amd as nw
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    h = vp_stream(stream)
    vp = ctypes.c_void_p
    calls_per_trial, trials = 200, 5
    cases = [(1, s) for s in synth.workload(1)] + [(2, s) for s in synth.workload(2)]
    cases += [(3, s) for s in synth.workload(3)]
    cases += [(4, s) for b in (1, 2, 4, 8) for s in synth.workload(4, batch=b)]
    out = []
    for wl, spec in cases:
        index = [s.name for s in synth.workload(wl, batch=spec.batch)].index(spec.name)
        res = single_matrix_timing(spec, wl, index, args.seed, stream, calls_per_trial, trials, full=True)
        log(f"config {res}")
        out.append(res)
    # the 13B layer as a decoder layer issues it: one group launch per (q,k,v), (o), (gate,up), (down),
    # every layer-sized copy of the seven products read once per 200 launches
    specs3 = synth.workload(3)
    mats3 = []
    for i, spec in enumerate(specs3):
        m = synth.make_matrix(spec, seed=args.seed, workload=3, index=i)
        mats3.append(dict(
            spec=spec, nnz=int(m.col.size), packed=nw.pack(torch.from_numpy(m.codes).cuda(), spec.bits),
            lut=torch.from_numpy(m.lut.view(np.int16)).cuda(), rp=torch.from_numpy(m.row_ptr).cuda(),
            col=torch.from_numpy(m.col.view(np.int16)).cuda(), val=torch.from_numpy(m.val.view(np.int16)).cuda(),
            x=torch.from_numpy(m.x.view(np.int16)).cuda(),
            y=torch.empty(spec.rows, dtype=torch.int16, device="cuda")))
    layer_bytes = sum(nw.algorithmic_bytes(d["spec"].rows, d["spec"].cols, d["spec"].bits, d["nnz"], 1) for d in mats3)
    reps = max(1, -(-1024 * 2 ** 20 // layer_bytes))
    layers = [mats3] + [[dict(d, **{k: d[k].clone() for k in ("packed", "lut", "rp", "col", "val")}) for d in mats3]
                        for _ in range(reps - 1)]
    levels = WeightStream.LEVELS
    descs = []
    for ms in layers:
        for lv in levels:
            arr = (nw.Product * len(lv))()
            for k, i in enumerate(lv):
                d = ms[i]
                arr[k] = nw.Product(d["packed"].data_ptr(), d["lut"].data_ptr(), d["rp"].data_ptr(), d["col"].data_ptr(),
                                    d["val"].data_ptr(), d["nnz"], d["spec"].rows, d["spec"].cols, d["x"].data_ptr(),
                                    d["y"].data_ptr())
            descs.append((arr, len(lv)))
    gws = torch.zeros(max(int(nw.library().sqllm_group_workspace_bytes(a, n, 1)) for a, n in descs), dtype=torch.uint8,
                      device="cuda")
    gfn = nw.library().sqllm_dense_sparse_gemv_group
    n_layers = 50
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for k in range(n_layers * len(levels)):
            arr, n = descs[k % len(descs)]
            st = gfn(arr, n, 3, 1, vp(gws.data_ptr()), gws.numel(), h)
            if st != 0:
                raise RuntimeError(f"sqllm_dense_sparse_gemv_group failed with status {st}")
    ts = []
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / n_layers)
    layer_us = statistics.median(ts)
    log(f"config 13B layer as four group launches: {layer_us:.2f} us, {layer_bytes / (layer_us * 1e3):.1f} GB/s")
    del g, layers, descs, mats3
    torch.cuda.empty_cache()

    totals = {}
    for wl, name in ((2, "mlp_pair"), (3, "layer")):
        sel = [r for r in out if r["workload"] == wl]
        us = sum(r["graph_us"] for r in sel)
        totals[f"workload{wl}_{name}"] = {"graph_us": round(us, 3), "GB_per_s": round(
            sum(r["bytes"] for r in sel) / (us * 1e3), 1)}
    totals["workload3_layer_group_launches"] = {"graph_us": round(layer_us, 3),
                                                "GB_per_s": round(layer_bytes / (layer_us * 1e3), 1)}
    print(json.dumps({"ablation": "configs", "unit": "us per product (median of 5 trials of 200 calls)",
                      "products": out, "totals": totals}), flush=True)


def offline_ablation(args) -> None:
    """The offline steps on the three LLaMA-65B shapes: thresholds (0.2 / 99.8
    percentiles and the 0.05% most sensitive), CSR + D extraction, and 3-bit
    weighted k-means (20 steps) of D.  Inputs: Student-t (4 degrees of
    freedom) weights x 0.02 and squared-normal sensitivities, drawn on the
    GPU from a seeded generator.  The split calls synchronise, so they are
    timed by the host clock around the call; the k-means by HIP events.  The
    oracle runs the same steps on a slice (split: 512 rows; k-means: 8 rows)
    of the 8192 x 8192 shape, scaled to the whole matrix by rows."""
    import numpy as np
    import torch

    import non_uniform_weight_amd as nw

    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed + 1234)
    shapes = [(8192, 8192, 4), (22016, 8192, 2), (8192, 22016, 1)]
    res, layer_ms = [], 0.0
    for rows, cols, count in shapes:
        z = torch.randn((rows, cols), device="cuda", generator=gen)
        chi = sum(torch.randn((rows, cols), device="cuda", generator=gen) ** 2 for _ in range(4)) / 4
        w = (0.02 * z / chi.sqrt()).half()
        del z, chi
        g = torch.randn((rows, cols), device="cuda", generator=gen)
        sens = (g * g).float()
        del g
        t = {}
        for rep in range(3):                       # the first pass warms up; the last is kept
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            t_min, t_max, t_s, nnz = nw.outlier_thresholds(w, 2000, sens, 500)
            t1 = time.perf_counter()
            rp, col, val, dense, sdense = nw.outlier_extract(w, t_min, t_max, nnz, sens, t_s)
            t2 = time.perf_counter()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            codes, lut = nw.kmeans_lut(dense, 3, 20, sdense)
            e1.record()
            torch.cuda.synchronize()
            t = {"thresholds_ms": (t1 - t0) * 1e3, "extract_ms": (t2 - t1) * 1e3,
                 "kmeans_ms": e0.elapsed_time(e1)}
        total = sum(t.values())
        layer_ms += count * total
        r = {"shape": f"{rows}x{cols}", "per_layer": count, "nnz": nnz, "density_pct": round(100 * nnz / (rows * cols), 4),
             **{k: round(v, 3) for k, v in t.items()}, "total_ms": round(total, 3),
             "kmeans_weight_steps_per_s": round(rows * cols * 20 / (t["kmeans_ms"] * 1e-3) / 1e9, 1)}
        log(f"offline {r}")
        res.append(r)
        if rows == cols:
            sample = (w[:512].cpu(), sens[:512].cpu(), dense[:8].cpu(), sdense[:8].cpu(), rows)
        del w, sens, rp, col, val, dense, sdense, codes, lut
        torch.cuda.empty_cache()
    out = {"ablation": "offline", "workload": "LLaMA-65B layer: 8192x8192 x4, 22016x8192 x2, 8192x22016 x1; "
           "0.4% outliers + 0.05% sensitive values; 3-bit weighted k-means, 20 steps", "shapes": res,
           "layer_ms": round(layer_ms, 2), "model_80_layers_s": round(80 * layer_ms / 1e3, 2)}
    if not args.no_cpu_baseline:
        from oracle import quantize as q
        w_s, s_s, d_s, sd_s, rows = sample
        wb = w_s.view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        t_min, t_max, t_s, _ = q.split_thresholds(wb, 2000, s_s.numpy(), 500)
        q.extract(wb, t_min, t_max, s_s.numpy(), t_s)
        t1 = time.perf_counter()
        q.kmeans_lut(d_s.view(torch.int16).numpy().view(np.uint16), sd_s.numpy(), 3, 20)
        t2 = time.perf_counter()
        split_ms = (t1 - t0) * 1e3 * rows / 512
        km_ms = (t2 - t1) * 1e3 * rows / 8
        out["cpu_baseline"] = {"kind": "oracle", "cores": 1, "unit": "ms per 8192x8192 matrix",
                               "split_ms": round(split_ms, 1), "kmeans_ms": round(km_ms, 1),
                               "sample": "split of rows 0-511 (thresholds over the slice) and k-means of rows 0-7, "
                                         "scaled by rows"}
    print(json.dumps(out), flush=True)


def launch_ceiling(args, reps: int) -> dict:
    """The launch structure's ceiling: one step of the stream as the same 320
    dependent launches (per layer (q,k,v), (o), (gate,up), (down)), each a
    plain read of exactly that launch's algorithmic bytes (rounded down to
    1 KiB) with no decode or arithmetic (sqllm_test_stream_read), captured in
    one HIP graph; and the same bytes as one launch."""
    import torch

    import non_uniform_weight_amd as nw
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    specs = synth.workload(5, bits=args.bits, density_bp=args.density_bp)[:7 * args.layers]
    sizes = []
    for l0 in range(0, len(specs), 7):
        for lv in WeightStream.LEVELS:
            b = sum(nw.algorithmic_bytes(specs[l0 + i].rows, specs[l0 + i].cols, specs[l0 + i].bits,
                                         specs[l0 + i].nnz, 1) for i in lv)
            sizes.append(b // 1024 * 1024)
    total = sum(sizes)
    buf = torch.ones(total, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    lib, h = nw.library(), vp_stream(stream)
    base = buf.data_ptr()

    def step_fn():
        off = 0
        for n in sizes:
            st = lib.sqllm_test_stream_read(base + off, n, sink.data_ptr(), h)
            if st != 0:
                raise RuntimeError(f"sqllm_test_stream_read failed with status {st}")
            off += n

    def timed(fn, reps):
        with torch.cuda.stream(stream):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step_fn()
    ms_graph = timed(g.replay, reps)
    ms_one = timed(lambda: lib.sqllm_test_stream_read(base, total, sink.data_ptr(), h), reps)
    del g, buf
    torch.cuda.empty_cache()
    out = {"launches_per_step": len(sizes), "bytes_per_step": total,
           "launches_as_reads": {"ms_per_step": round(ms_graph, 4), "GB_per_s": round(total / ms_graph / 1e6, 1),
                                 "frac": round(total / ms_graph / 1e6 / HBM_PEAK_GBS, 4),
                                 "us_per_launch": round(ms_graph * 1e3 / len(sizes), 3)},
           "one_read": {"ms": round(ms_one, 4), "GB_per_s": round(total / ms_one / 1e6, 1),
                        "frac": round(total / ms_one / 1e6 / HBM_PEAK_GBS, 4)}}
    log(f"ceiling: {len(sizes)} reads {ms_graph:.3f} ms ({total / ms_graph / 1e6:.0f} GB/s), one read {ms_one:.3f} ms "
        f"({total / ms_one / 1e6:.0f} GB/s)")
    return out


def ceiling_ablation(args) -> None:
    print(json.dumps(dict(ablation="ceiling", **launch_ceiling(args, args.steps))), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the design notes describe row sharding across GPUs).", file=sys.stderr)
        sys.exit(2)
    if args.ablation == "outliers":
        outlier_ablation(args)
        return
    if args.ablation == "batch":
        batch_ablation(args)
        return
    if args.ablation == "offline":
        offline_ablation(args)
        return
    if args.ablation == "configs":
        config_table(args)
        return
    if args.ablation == "ceiling":
        ceiling_ablation(args)
        return
    import torch

    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    specs = synth.workload(5, bits=args.bits, density_bp=args.density_bp)[:7 * args.layers]
    ws = WeightStream(specs, args.seed)
    n_products = len(ws.calls)
    stream = torch.cuda.Stream()

    def time_mode(step_fn):
        """ms per step: W warm-up steps, then K timed steps between events on
        the launch stream; one step = every product of the stream, launched
        back to back, captured once in a HIP graph (plain launches with
        --no-graph)."""
        def run_step():
            step_fn(stream)

        if not args.no_graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step_fn(stream)
            run_step = g.replay
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            for _ in range(args.warmup):
                run_step()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                run_step()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    mode = "plain launches" if args.no_graph else "HIP graph replay"
    single_ms = None
    if not (args.no_single and args.launch == "level"):
        single_ms = time_mode(ws.step)
        log(f"single calls, {mode}: {single_ms:.3f} ms/step ({single_ms * 1e3 / n_products:.2f} us/product)")
    if args.launch == "level":
        ms = time_mode(ws.step_grouped)
        n_launches = len(ws.groups)
        # (q,k,v) and (gate,up) run dense_sparse_group_kernel, the one-product levels (o) and (down)
        # dense_sparse_kernel: one kernel body, its arguments from a per-product table or passed directly
        kernel = f"dense_sparse{{,_group}}_kernel<{args.bits},1,fused,matrix>"
        log(f"group launches, {mode}: {ms:.3f} ms/step ({n_launches} launches)")
    else:
        # 22016x8192 (344 row tiles) runs as two row slices in one group launch
        ms, n_launches = single_ms, n_products
        kernel = (f"dense_sparse_kernel<{args.bits},1,fused,matrix>, 22016-row products "
                  f"dense_sparse_group_kernel<{args.bits},1,fused,matrix>")

    bytes_per_step = ws.bytes_per_step
    value = bytes_per_step / (ms * 1e-3) / 1e9
    # level launches all run the group kernel; its average duration is the
    # timed region's length over the launches in it
    avg_launch_ms = ms / n_launches
    avg_bytes = bytes_per_step / n_launches
    achieved = avg_bytes / (avg_launch_ms * 1e-3) / 1e9
    log(f"per launch: {avg_launch_ms * 1e3:.2f} us avg, {achieved:.0f} GB/s")
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    traffic = measured_traffic(kernel) if args.bits == 3 and args.density_bp == 45 else None
    del ws
    torch.cuda.empty_cache()
    matrices = None if args.no_per_matrix else per_matrix(args.seed, stream)
    ceiling = None if args.no_per_matrix else launch_ceiling(args, 20)
    cpu = None
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(specs, args.seed, threads)
        log(f"cpu baseline: {cpu['value']} GB/s with {threads} threads")

    out = {
        "metric": f"effective HBM GB/s (% of peak) and \u00b5s/GEMV, {args.bits}-bit LUT+sparse, batch 1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"80-layer LLaMA-65B-shaped weight stream, {n_products} GEMVs "
                        f"(8192x8192 x4, 22016x8192 x2, 8192x22016 per layer), {args.bits}-bit codes, "
                        f"{args.density_bp / 100:.2f}% uniform CSR outliers, batch 1",
            "bits": args.bits,
            "outlier_density_pct": args.density_bp / 100,
            "batch": 1,
            "gemvs_per_step": n_products,
            "bytes_per_step": bytes_per_step,
            "launch": mode + (", one group launch per (q,k,v), (o), (gate,up), (down)" if args.launch == "level"
                              else ", one call per product"),
        },
        "us_per_gemv": round(ms * 1e3 / n_products, 3),
        "single_calls": None if single_ms is None else {
            "value": round(bytes_per_step / (single_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "us_per_gemv": round(single_ms * 1e3 / n_products, 3)},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "launches_per_step": n_launches,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": round(avg_bytes),
        },
        "per_matrix": matrices,
        # the same launches as plain reads of the same bytes, no arithmetic: what any kernel could reach with
        # this launch structure
        "launch_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
