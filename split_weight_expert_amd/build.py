"""Build libdwdp.so (gfx950) in place: every csrc/*.hip and csrc/*.cpp through hipcc.

Another build of the same sources (compile-time options in DWDP_EXTRA_FLAGS) goes elsewhere with
--out, e.g. the tile-trace build that bench.py --tile-trace loads through DWDP_LIBRARY:

    DWDP_EXTRA_FLAGS=-DDWDP_TILE_TRACE=1 python split_weight_expert_amd/build.py \
        --out split_weight_expert_amd/lib/trace/libdwdp.so
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libdwdp.so")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build", "dwdp")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics"]


def _compile(src: str, objdir: str, defines: list[str]) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    # DWDP_EXTRA_FLAGS: compile-time options of the kernels (e.g. -DDWDP_FP8_BM256), space separated
    extra = os.environ.get("DWDP_EXTRA_FLAGS", "").split() + defines
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


# The tile-trace build (bench.py --tile-trace, tests/test_gpu_diag.py): the same sources with
# -DDWDP_TILE_TRACE=1, beside the default library.
TRACE_LIB = os.path.join(LIBDIR, "trace", "libdwdp.so")
TRACE_DEFINES = ["-DDWDP_TILE_TRACE=1"]


def build(verbose: bool = False, out: str | None = None, defines: list[str] | None = None) -> str:
    lib = os.path.abspath(out) if out else LIB
    # objects of another build go to a folder of their own, so that builds never mix
    objdir = OBJDIR if lib == LIB else OBJDIR + "-" + hashlib.sha1(lib.encode()).hexdigest()[:12]
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, list(defines or [])), srcs))
    tmp = lib + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=None, help="library path (default: lib/libdwdp.so next to this script)")
    build(verbose=True, out=ap.parse_args().out)
