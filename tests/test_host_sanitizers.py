"""The library's host-only logic under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

split_weight_expert_amd/csrc/host.cpp -- the round-robin slice plan of the prefetch, the expert
record layout, the pointer table over split buffers and the workspace sizing -- is built with g++
and -fsanitize=address,undefined together with a randomised driver (tests/host_sanitize/
fuzz_host.cpp) that checks the plan covers every byte once in round-robin order, the table points
at the right record parts, invalid arguments are rejected and no output array is overrun.  Any
sanitizer report aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "split_weight_expert_amd", "csrc", "host.cpp"),
       os.path.join(ROOT, "tests", "host_sanitize", "fuzz_host.cpp")]


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    out = str(tmp_path_factory.mktemp("asan") / "fuzz_host")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", *SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_logic_under_sanitizers(fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_bin, str(seed), "1500"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host logic ok" in r.stdout
