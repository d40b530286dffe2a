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


@pytest.mark.parametrize("seed", range(6))
def test_burst_parts_are_the_plan_cut_by_rounds(seed):
    """--burst-at releases parts of the slice plan; planned one after another they must give exactly the
    oracle's round-robin plan of the whole copy (same slices, same order)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from oracle.prefetch import chunk_plan
    rng = np.random.default_rng(seed)
    chunk = int(rng.choice([16, 48, 4096]))
    n_src = int(rng.integers(1, 5))
    sizes = [int(rng.integers(0, 20 * chunk)) for _ in range(n_src)]
    bases = [0x100000 * (s + 1) for s in range(n_src)]
    offs = list(np.cumsum([0] + sizes[:-1]))
    sources = [(b, int(o), n) for b, o, n in zip(bases, offs, sizes)]

    def plan(srcs):
        return [(srcs[s][0] + so, do, ln) for s, so, do, ln in chunk_plan([x[2] for x in srcs], [x[1] for x in srcs],
                                                                            chunk)]
    whole = plan(sources)
    for n in (1, 2, 3, 5):
        got = [sl for part in bench.burst_parts(sources, chunk, n) for sl in plan(part)]
        assert got == whole, (n, sizes, chunk)
