"""bench.py's command-line contract, checked without a GPU.

One GPU only: --gpus above 1 exits with status 2 and says so, before anything touches the GPU.
The options the measurement legs use parse to the values they are given.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _bench("--gpus", n, "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_options_parse(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "prefill16k_fp8", "--copy-engine", "sdma",
                                      "--copy-workgroups", "24", "--copy-streams", "2", "--chunk-mib", "1",
                                      "--shape-study", "--pipeline-layers", "3", "--no-cpu-baseline"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup) == (1, 20, 3)
    assert a.workload == "prefill16k_fp8" and a.copy_engine == "sdma"
    assert (a.copy_workgroups, a.copy_streams, a.chunk_mib, a.pipeline_layers) == (24, 2, 1.0, 3)
    assert a.shape_study and a.no_cpu_baseline and not a.no_prefetch
