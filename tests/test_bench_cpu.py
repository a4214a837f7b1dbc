"""The benchmark's command-line contract, without a GPU (CPU only)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=timeout, cwd=ROOT)


@pytest.mark.parametrize("extra", [[], ["--ablation", "configs"]])
def test_more_than_one_gpu_is_refused_with_a_message(extra):
    r = _run("--gpus", "2", *extra)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_without_a_gpu_the_bench_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "no GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = _run("--help", timeout=60)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--bits", "--density-bp", "--ablation", "--no-single"):
        assert flag in r.stdout
