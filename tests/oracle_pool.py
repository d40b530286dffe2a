"""The oracle evaluated in worker processes (test infrastructure only): the per-expert FFN, and the
E4M3 codec over ranges of fp32 bit patterns.

A full-size layer's oracle output for a few hundred tokens needs most of the 256 experts' weights:
generating them, and for fp8 block-quantising them, takes seconds per expert on one core.  This
module runs the same oracle functions that oracle.moe.moe_layer runs for one expert -- generate the
weights, prepare_weights, prepare_tokens, expert_ffn -- in a pool of spawned processes, one expert
per task, and the caller combines the rows with oracle.moe.combine exactly as moe_layer does.

It imports neither torch nor the package, so the workers never touch the GPU; each worker keeps
its BLAS to one thread.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np


def _init_worker():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass


def expert_rows(cfg, e: int, x_rows: np.ndarray, layer: int = 0, parts: bool = False, with_wd: bool = False,
                precision: str | None = None):
    """Oracle outputs of expert e (e == E: the shared expert) for the given token rows (float32 [n, H]):
    Y [n, H] float64, or the full expert_ffn_parts dict when parts (with the prepared down weights
    under "wd" when with_wd).  precision overrides the workload's policy (e.g. "f32": the unquantised,
    unrounded fp64 FFN of the same generated weights)."""
    import synth
    from oracle import moe
    pol = precision or cfg.dtype
    wts = moe.prepare_weights(*synth.expert_weights(cfg, e, layer), pol)
    X = moe.prepare_tokens(x_rows, pol)
    if parts:
        p = moe.expert_ffn_parts(X, *wts, pol)
        if with_wd:
            p["wd"] = wts[2]
        return p
    return moe.expert_ffn(X, *wts, pol)


def _task(args):
    cfg, e, rows, layer, parts, with_wd, precision = args
    return e, expert_rows(cfg, e, rows, layer, parts, with_wd, precision)


def pool_size() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def map_experts(cfg, jobs, layer: int = 0, parts: bool = False, with_wd=(), timeout: float = 900.0,
                precision: str | None = None):
    """jobs: {expert: token rows float32 [n, H]} -> {expert: oracle result}, evaluated in parallel.

    Workers are spawned (they re-import the caller's main module by name, so the caller must be an
    importable program such as pytest, not a script read from stdin); `timeout` bounds the whole map.
    with_wd: experts whose prepared down weights are returned too (parts only)."""
    order = sorted(jobs, key=lambda e: -len(jobs[e]))
    ctx = mp.get_context("spawn")
    out = {}
    with cf.ProcessPoolExecutor(max_workers=min(pool_size(), max(1, len(order))), mp_context=ctx,
                                initializer=_init_worker) as ex:
        for e, res in ex.map(_task, [(cfg, e, jobs[e], layer, parts, e in with_wd, precision) for e in order],
                             timeout=timeout):
            out[e] = res
    return out


def layer_outputs(cfg, x, idx, w, tokens, layer: int = 0):
    """The oracle's block output y for `tokens` under the routing (idx, w), as oracle.moe.moe_layer
    computes it: every chosen expert's FFN of the token's row, summed with the gate weights in slot
    order, then the shared expert's row, with the precision policy's one final rounding."""
    from oracle import moe
    tokens = [int(t) for t in tokens]
    jobs = {}
    for t in tokens:
        for j in range(idx.shape[1]):
            jobs.setdefault(int(idx[t, j]), []).append(t)
    if cfg.shared:
        jobs[cfg.E] = list(tokens)
    uniq = {e: sorted(set(ts)) for e, ts in jobs.items()}
    res = map_experts(cfg, {e: x[np.asarray(ts)] for e, ts in uniq.items()}, layer)
    pos = {e: {t: i for i, t in enumerate(ts)} for e, ts in uniq.items()}
    y = np.zeros((len(tokens), x.shape[1]))
    for i, t in enumerate(tokens):
        rows = np.stack([res[int(idx[t, j])][pos[int(idx[t, j])][t]] for j in range(idx.shape[1])])
        sh = res[cfg.E][pos[cfg.E][t]] if cfg.shared else None
        y[i] = moe.combine(rows, w[t], sh, cfg.dtype)
    return y


def _e4m3_task(args):
    lo, hi, sign = args
    from oracle import codecs
    bits = np.arange(lo, hi, dtype=np.uint32) | np.uint32(sign)
    return codecs.e4m3_encode(bits.view(np.float32))


def e4m3_codes(lo: int, hi: int, sign: int, ex, parts: int = 16, timeout: float = 300.0) -> np.ndarray:
    """The oracle's E4M3 codes of the fp32 bit patterns lo .. hi-1 (each OR-ed with sign), computed in
    `parts` tasks on the executor ex (a pool from e4m3_pool())."""
    cuts = [lo + (hi - lo) * i // parts for i in range(parts + 1)]
    tasks = [(a, b, sign) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    return np.concatenate(list(ex.map(_e4m3_task, tasks, timeout=timeout)))


def _bf16_task(args):
    lo, hi = args
    from oracle import codecs
    v = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)
    return codecs.bf16_bits(0.0 + v)          # a sum that starts at +0, as the combine's does


def bf16_codes(lo: int, hi: int, ex, parts: int = 16, timeout: float = 300.0) -> np.ndarray:
    """bf16 storage bits of the oracle's rounding of 0 + x for the fp32 bit patterns x = lo .. hi-1."""
    cuts = [lo + (hi - lo) * i // parts for i in range(parts + 1)]
    tasks = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    return np.concatenate(list(ex.map(_bf16_task, tasks, timeout=timeout)))


def e4m3_pool():
    """A pool of spawned CPU workers for e4m3_codes and bf16_codes (use as a context manager)."""
    return cf.ProcessPoolExecutor(max_workers=pool_size(), mp_context=mp.get_context("spawn"),
                                  initializer=_init_worker)
