"""Host checks of bench.py's command line (no GPU needed): it measures one
GPU only and refuses other counts with a message, and fails loudly (not
with a CPU number) when no GPU is visible."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is visible")
def test_no_gpu_fails_without_a_number():
    r = run("--steps", "1", "--warmup", "1")
    assert r.returncode == 3
    assert "no GPU" in r.stderr
    assert r.stdout == ""


def test_every_workload_is_selectable():
    r = run("--help")
    assert r.returncode == 0
    for name in ("gqa_causal_bf16", "splitd_bf16_d1024", "fp8_outlier", "bwd_causal_bf16"):
        assert name in r.stdout
