"""Build the two synthetic-input generator libraries in place (gcc for the host, hipcc for gfx950)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    host_src = os.path.join(HERE, "synth_host.c")
    host_out = os.path.join(HERE, "libsynth_host.so")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    host_src, "-o", host_out], check=True, capture_output=not verbose)
    gpu_src = os.path.join(HERE, "synth_gpu.hip")
    gpu_out = os.path.join(HERE, "libsynth_gpu.so")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.run([hipcc, *HIP_FLAGS, gpu_src, "-o", gpu_out], check=True, capture_output=not verbose)


if __name__ == "__main__":
    build(verbose=True)
