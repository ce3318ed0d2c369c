"""CPU: bench.py's command-line contract where no GPU work is involved -- one
GPU only, and a clear exit when no GPU is visible."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    res = run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU only" in line["error"]


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is visible here")
def test_no_gpu_exits_nonzero_without_a_json_line():
    res = run("--steps", "1", "--warmup", "0")
    assert res.returncode == 3
    assert "no GPU visible" in res.stderr
    assert not res.stdout.strip()
