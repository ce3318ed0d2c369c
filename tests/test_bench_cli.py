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


def test_profiles_count_only_while_they_match_the_sources(tmp_path):
    # bench.py takes the M=1 kernel times and the M=256 traffic from the
    # committed summaries only while their source hash is the current one
    sys.path.insert(0, ROOT)
    import bench

    eager, graph, counters = (tmp_path / n for n in ("eager.json", "graph.json", "counters.json"))
    eager.write_text(json.dumps({"kernel_source_sha256_16": "aaaa", "median_us": 3.3, "calls": 10,
                                 "kernel": "k"}))
    graph.write_text(json.dumps({"kernel_source_sha256_16": "bbbb", "median_us": 3.1, "calls": 10,
                                 "kernel": "k"}))
    counters.write_text(json.dumps({"kernel_source_sha256_16": "aaaa", "variant": "fused",
                                    "traffic_bytes_per_launch": 419869616}))
    paths = {"eager": str(eager), "graph": str(graph), "missing": str(tmp_path / "none.json")}
    m1, traffic = bench.current_profiles(paths, str(counters), "fused", "aaaa")
    assert set(m1) == {"eager"} and m1["eager"]["median_us"] == 3.3 and traffic == 419869616
    m1, traffic = bench.current_profiles(paths, str(counters), "split", "aaaa")
    assert traffic is None  # counters of the other variant
    m1, traffic = bench.current_profiles(paths, str(counters), "fused", "cccc")
    assert m1 == {} and traffic is None
