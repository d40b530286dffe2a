"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Each case builds the whole synthetic layer on the GPU (DeviceLayer: 64 resident
experts + the shared expert, 192 in a prefetch slot set) and runs route ->
permute -> GEMM1+SwiGLU -> GEMM2 -> combine exactly as bench.py does.  Then:

* routing in full: the GPU's fp32 logits against the oracle's fp64 logits
  (<= 1e-5 relative to their rms), the GPU's indices equal to the oracle's
  top-k of those same logits (bit-exact), and its gate weights against the
  oracle's softmax over them;
* permutation in full: offsets, perm_src and inv_perm bit-exact against the
  oracle's stable permutation of the GPU's indices (GEMM1 reads the token
  rows through perm_src; for fp8, sampled tokens' codes and scales are
  bit-exact against the oracle's group quantiser);
* expert outputs y_perm on every row of at least 16 routed groups, chosen so
  that the last m-tiles of the groups cover every row count of the workload's
  routing that the expert GEMMs have a variant for (the smallest such groups
  first; all variants for the bf16 prefill workloads), and on 64 sampled rows
  of the shared expert's group, against the oracle's expert FFN of those rows
  (fp8: A's codes as well, allowing re-quantisation flips at rounding
  boundaries);
* block outputs y on 512 sampled tokens (bf16; all tokens of the 64-token
  decode batch) or 64 sampled tokens (fp8), computed by the oracle's expert
  FFNs and combine under the GPU's routing.
The oracle's per-expert work runs in a pool of CPU processes (tests/oracle_pool.py).
All floating-point checks use the dtype's tolerance.
"""
import time

import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe
from tests import oracle_pool
from tests.gpu_util import TOL, assert_close, check_fp8_rows, ffn_ws_a, need_gpu, rel_err, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_block(cfg):
    from split_weight_expert_amd.workload import DeviceLayer
    layer = DeviceLayer(cfg, "cuda", slot_sets=1)
    block = layer.block()
    b = block.buffers(cfg.T)
    table = layer.table(1)
    block.route(layer.x, layer.w_router, layer.bias, b)
    block.permute(layer.x, b)
    block.ffn_stage(1, table, b)
    block.ffn_stage(2, table, b)
    block.combine(b)
    torch.cuda.synchronize()
    return layer, b


def tile_rows(cfg, rows, groups):
    """The expert GEMMs' m-tile height for this shape (from the mean rows per group; fp8 at most 128
    unless the library was built with the 256-row fp8 tiles, which its version string names)."""
    from split_weight_expert_amd import api
    mean = rows // groups
    bm = 256 if mean >= 192 else 128 if mean >= 96 else 64 if mean >= 40 else 32
    return min(bm, 128) if cfg.dtype == "fp8" and "fp8-bm256" not in api.version() else bm


def pick_groups(counts, bm, per=2, at_least=16):
    """Routed groups whose last m-tile covers every active 32-row block count 1 .. bm/32, `per` groups
    each (the smallest first), topped up with the next smallest groups to at least `at_least`."""
    nz = [g for g in np.argsort(counts, kind="stable") if counts[g] > 0]
    by_tail = {}
    for g in nz:
        tail = (int(counts[g]) - 1) % bm + 1
        by_tail.setdefault((tail + 31) // 32, []).append(int(g))
    chosen = []
    for ma in range(1, bm // 32 + 1):
        chosen += by_tail.get(ma, [])[:per]
    for g in nz:
        if len(chosen) >= at_least:
            break
        if int(g) not in chosen:
            chosen.append(int(g))
    return sorted(set(chosen)), sorted(by_tail)


def sample_tokens(idx, counts, T, n):
    if n >= T:
        return list(range(T))
    big = int(np.argmax(counts))
    nz = np.flatnonzero(counts)
    small = int(nz[np.argmin(counts[nz])])
    t_big = int(np.flatnonzero((idx == big).any(1))[0])
    t_small = int(np.flatnonzero((idx == small).any(1))[-1])
    even = np.linspace(0, T - 1, max(n - 4, 0) + 2).astype(int)[1:-1]
    out = sorted({0, T - 1, t_big, t_small, *map(int, even)})
    extra = iter(t for t in range(T) if t not in set(out))
    while len(out) < n:
        out.append(next(extra))
    return sorted(out)


def _token_jobs(toks, idx, cfg):
    """expert -> the sampled tokens it computes (their k chosen experts and the shared expert)."""
    jobs = {}
    for t in toks:
        for j in range(cfg.k):
            jobs.setdefault(int(idx[t, j]), []).append(int(t))
        if cfg.shared:
            jobs.setdefault(cfg.E, []).append(int(t))
    return jobs


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name,n_tokens", [
    ("prefill8k_bf16", 512),
    ("imbalanced_bf16", 512),
    ("decode64_bf16", 64),
    ("prefill16k_fp8", 64),
])
def test_full_size_block(name, n_tokens):
    cfg = synth.get_config(name)
    t0 = time.time()
    print(f"\n[full-size] {name}: T={cfg.T} dtype={cfg.dtype}", flush=True)
    layer, b = run_block(cfg)
    print(f"[full-size] {name}: block done ({time.time() - t0:.0f} s)", flush=True)

    # ---- routing, all tokens
    x = synth.tokens(cfg)
    wr = synth.router_weight(cfg)
    bias = synth.router_bias(cfg)
    lo = omoe.router_logits(x, wr, bias)
    lg = b.logits.cpu().numpy()
    rms = np.sqrt((lo ** 2).mean())
    assert np.abs(lg - lo).max() <= 1e-5 * rms, "router logits"
    idx = b.idx.cpu().numpy()
    np.testing.assert_array_equal(idx, omoe.topk_select(lg, cfg.k))
    w = b.w.cpu().numpy()
    gw = omoe.gate_weights(lg, idx)
    np.testing.assert_allclose(w, gw, rtol=2e-6, atol=1e-7)

    # ---- permutation, all rows
    offsets, perm_src, inv_perm, counts = omoe.permute(idx, cfg.E, cfg.shared)
    np.testing.assert_array_equal(b.offsets.cpu().numpy(), offsets)
    np.testing.assert_array_equal(b.perm_src.cpu().numpy(), perm_src)
    np.testing.assert_array_equal(b.inv_perm.cpu().numpy(), inv_perm)
    gc = np.diff(offsets)                                   # rows per group, the shared group included
    if cfg.dtype == "fp8":
        # the tokens GEMM1 reads: per-token codes and scales, bit-exact (sampled tokens)
        toks_q = np.unique(np.concatenate([[0, cfg.T - 1], perm_src[offsets[:-1][gc > 0]],
                                           np.linspace(0, cfg.T - 1, 64).astype(int)]))
        sel = torch.from_numpy(toks_q).cuda()
        q, s = omoe.quantize_groups(x[toks_q].astype(np.float32))
        np.testing.assert_array_equal(b.x_q[sel].cpu().numpy(), q)
        np.testing.assert_array_equal(b.x_q_scale[sel].cpu().numpy(), s)
    print(f"[full-size] {name}: routing and permutation bit-exact ({time.time() - t0:.0f} s)", flush=True)

    # ---- what the oracle evaluates: all rows of the chosen groups, sampled shared rows, sampled tokens
    G = cfg.E + cfg.shared
    bm = tile_rows(cfg, len(perm_src), G)
    groups, tails = pick_groups(counts, bm)
    assert len(groups) >= 16
    # pick_groups takes every tail variant the workload's routing produces (the balanced 16K-token fp8
    # routing gives only some; the deep-K grouped FFN test covers every variant)
    if cfg.dtype == "bf16" and bm == 256:
        assert tails == list(range(1, bm // 32 + 1)), f"tail variants present: {tails}"
    toks = sample_tokens(idx, counts, cfg.T, n_tokens)
    jobs = {}
    for g in groups:
        jobs.setdefault(g, set()).update(perm_src[offsets[g]:offsets[g + 1]].tolist())
    sh_rows = None
    if cfg.shared:
        sh_rows = np.unique(np.linspace(offsets[cfg.E], offsets[cfg.E + 1] - 1, min(64, cfg.T)).astype(int))
        jobs.setdefault(cfg.E, set()).update(perm_src[sh_rows].tolist())
        jobs[cfg.E].update(toks)
    for t in toks:
        for j in range(cfg.k):
            jobs.setdefault(int(idx[t, j]), set()).add(int(t))
    jobs = {e: np.array(sorted(ts)) for e, ts in jobs.items()}
    print(f"[full-size] {name}: oracle over {len(jobs)} experts, {sum(len(v) for v in jobs.values())} token "
          f"rows, {oracle_pool.pool_size()} processes", flush=True)
    fp8 = cfg.dtype == "fp8"
    res = oracle_pool.map_experts(cfg, {e: x[ts] for e, ts in jobs.items()}, parts=fp8,
                                  with_wd=set(groups) | {cfg.E})
    pos = {e: {int(t): i for i, t in enumerate(ts)} for e, ts in jobs.items()}
    print(f"[full-size] {name}: oracle done ({time.time() - t0:.0f} s)", flush=True)

    def ref_rows(e, tokens, key="Y"):
        r = res[e][key] if fp8 else res[e]
        return r[[pos[e][int(t)] for t in tokens]]

    # ---- expert rows: every row of the chosen groups, sampled rows of the shared group
    checks = [(g, np.arange(offsets[g], offsets[g + 1])) for g in groups]
    if cfg.shared:
        checks.append((cfg.E, sh_rows))
    stats = {}
    for g, rws in checks:
        got = to_np(b.y_perm[torch.from_numpy(rws).cuda()])
        tk = perm_src[rws]
        what = f"{name} group {g} ({gc[g]} rows, {len(rws)} compared)"
        if fp8:
            parts = {k_: ref_rows(g, tk, k_) for k_ in ("Y", "A", "A_pre", "A_codes", "A_scales")}
            codes, scales = ffn_ws_a(b.ws_ffn, len(perm_src), cfg.I, rws)
            check_fp8_rows(got, codes, scales, parts, res[g]["wd"], np.sqrt((parts["Y"] ** 2).mean()), what, stats)
            mx, mn = rel_err(got, parts["Y"])
            assert mn <= TOL["fp8"]["mean"], f"{what}: mean rel {mn:.2e}"
        else:
            mx, mn = assert_close(got, ref_rows(g, tk), cfg.dtype, what)
    print(f"[full-size] {name}: {len(checks)} groups' rows ok (tile {bm} rows, tails {tails})"
          + (f"; A codes {stats['codes']}, flips {stats['flips']} ({stats['flips'] / stats['codes']:.1e}), "
             f"worst flip {stats['worst_window']:.3f} windows, scales within {stats['scale_rel_max']:.1e}" if fp8
             else ""), flush=True)

    # ---- block outputs on the sampled tokens, combined as the oracle's layer combines them
    y = to_np(b.y[torch.tensor(toks).cuda()])
    ref = np.zeros_like(y, dtype=np.float64)
    for i, t in enumerate(toks):
        rows = np.stack([ref_rows(int(idx[t, j]), [t])[0] for j in range(cfg.k)])
        sh = ref_rows(cfg.E, [t])[0] if cfg.shared else None
        ref[i] = omoe.combine(rows, gw[t], sh, cfg.dtype)
    mx, mn = assert_close(y, ref, cfg.dtype, f"{name} {len(toks)} sampled tokens")
    print(f"[full-size] {name}: {len(toks)} tokens max rel {mx:.2e} mean rel {mn:.2e} ({time.time() - t0:.0f} s)",
          flush=True)

    # ---- the same tokens against unquantised, unrounded math (the oracle's fp64 FFN of the generated
    # weights and the token values, same routing): the error the precision policy itself costs.  Reported,
    # with only a coarse bar that catches a broken path.
    tj = {e: np.array(sorted(set(ts))) for e, ts in _token_jobs(toks, idx, cfg).items()}
    uq = oracle_pool.map_experts(cfg, {e: x[ts] for e, ts in tj.items()}, precision="f32")
    upos = {e: {int(t): i for i, t in enumerate(ts)} for e, ts in tj.items()}
    exact = np.zeros_like(y, dtype=np.float64)
    for i, t in enumerate(toks):
        rows = np.stack([uq[int(idx[t, j])][upos[int(idx[t, j])][t]] for j in range(cfg.k)])
        sh = uq[cfg.E][upos[cfg.E][t]] if cfg.shared else None
        exact[i] = omoe.combine(rows, gw[t], sh, "f32")
    emx, emn = rel_err(y, exact)
    print(f"[full-size] {name}: against unquantised fp64 math: max rel {emx:.2e} mean rel {emn:.2e}", flush=True)
    assert emn <= (0.1 if cfg.dtype == "fp8" else 1e-2), f"{name}: mean rel {emn:.2e} against unquantised math"
