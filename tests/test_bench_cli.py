"""bench.py's command-line contract that holds without a GPU (CPU only)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300,
                          env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_a_rank_of_a_multi_process_launch_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _run(env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_gpu_no_number():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert "needs the GPU" in r.stderr
    assert r.stdout == ""


def test_committed_summaries_carry_bench_data():
    # the counter summaries bench.py reads exist and hold a parseable data line
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_paths", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for path in (bench.TRAFFIC_SUMMARY, bench.GEMM_SUMMARY):
        with open(path) as f:
            lines = [ln for ln in f if ln.startswith("bench-data: ")]
        assert len(lines) == 1, path
        data = json.loads(lines[0][len("bench-data: "):])
        assert len(data["source_sha256"]) == 64


def test_committed_summaries_match_the_kernel_sources():
    # the counters behind roofline.traffic were taken on the sources in the tree:
    # a kernel change without new counters would leave the benchmark reporting
    # traffic null
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_paths", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    assert bench.summary_data(bench.TRAFFIC_SUMMARY, bench.KERNEL_SOURCES) is not None
    assert bench.summary_data(bench.GEMM_SUMMARY, bench.GEMM_SOURCES) is not None
