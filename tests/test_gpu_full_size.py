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
* expert outputs y_perm on sampled rows (first, last and evenly spaced) of
  the largest group, the smallest non-empty group and the shared expert's
  group, against the oracle's expert FFN of those rows;
* bf16 layers: block outputs y on a sample of tokens (the first, the last,
  tokens of the largest and of the smallest non-empty group, and evenly
  spaced ones), computed one expert at a time by the oracle under the GPU's
  routing.  fp8 layers instead check the combine of the GPU's own expert rows
  for sampled tokens, because the oracle's block quantiser needs seconds per
  expert and a token touches up to nine experts.
All floating-point checks use the dtype's tolerance.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe
from tests.gpu_util import assert_close, check_fp8_rows, ffn_ws_a, need_gpu, rel_err, to_np

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


def sample_tokens(idx, counts, T, n):
    big = int(np.argmax(counts))
    nz = np.flatnonzero(counts)
    small = int(nz[np.argmin(counts[nz])])
    t_big = int(np.flatnonzero((idx == big).any(1))[0])
    t_small = int(np.flatnonzero((idx == small).any(1))[-1])
    even = np.linspace(0, T - 1, max(n - 4, 0) + 2).astype(int)[1:-1]
    return sorted({0, T - 1, t_big, t_small, *map(int, even)})


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,n_tokens", [
    ("prefill8k_bf16", 6),
    ("imbalanced_bf16", 6),
    ("decode64_bf16", 6),
    ("prefill16k_fp8", 6),
])
def test_full_size_block(name, n_tokens):
    cfg = synth.get_config(name)
    print(f"\n[full-size] {name}: T={cfg.T} dtype={cfg.dtype}", flush=True)
    layer, b = run_block(cfg)

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
    np.testing.assert_allclose(w, omoe.gate_weights(lg, idx), rtol=2e-6, atol=1e-7)

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

    # ---- expert rows of sampled groups
    G = cfg.E + cfg.shared
    nz = np.flatnonzero(counts)
    groups = sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])} | ({cfg.E} if cfg.shared else set()))
    for g in groups:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        rws = np.unique(np.linspace(r0, r1 - 1, min(8, r1 - r0)).astype(int))
        wts = omoe.prepare_weights(*synth.expert_weights(cfg, g), cfg.dtype)
        parts = omoe.expert_ffn_parts(omoe.prepare_tokens(x[perm_src[rws]], cfg.dtype), *wts, cfg.dtype)
        got = to_np(b.y_perm[torch.from_numpy(rws).cuda()])
        what = f"{name} group {g} rows {rws.tolist()}"
        if cfg.dtype == "fp8":
            codes, scales = ffn_ws_a(b.ws_ffn, len(perm_src), cfg.I, rws)
            flips, mx = check_fp8_rows(got, codes, scales, parts, wts[2], np.sqrt((parts["Y"] ** 2).mean()), what)
            mn = rel_err(got, parts["Y"])[1]
        else:
            mx, mn = assert_close(got, parts["Y"], cfg.dtype, what)
        print(f"[full-size] {name}: group {g} ({r1 - r0} rows) max rel {mx:.2e} mean rel {mn:.2e}", flush=True)

    toks = sample_tokens(idx, counts, cfg.T, n_tokens)
    y = to_np(b.y[torch.tensor(toks).cuda()])
    gw = omoe.gate_weights(lg, idx)
    if cfg.dtype == "fp8":
        # the combine of the GPU's own expert rows, in full precision order
        yp = {t: to_np(b.y_perm[torch.from_numpy(inv_perm[t].astype(np.int64)).cuda()]) for t in toks}
        sh = to_np(b.y_perm[torch.tensor([cfg.T * cfg.k + t for t in toks]).cuda()]) if cfg.shared else None
        ref_y = np.stack([omoe.combine(yp[t], gw[t], None if sh is None else sh[i], cfg.dtype)
                          for i, t in enumerate(toks)])
        mx, mn = assert_close(y, ref_y, cfg.dtype, f"{name} combine of tokens {toks}")
    else:
        routing = (lg.astype(np.float64), idx, gw)
        ref = omoe.moe_layer(x, wr, bias, cfg.k, lambda e: synth.expert_weights(cfg, e),
                             (lambda: synth.expert_weights(cfg, cfg.E)) if cfg.shared else None,
                             precision=cfg.dtype, tokens=toks, routing=routing)
        mx, mn = assert_close(y, ref["y"], cfg.dtype, f"{name} sampled tokens {toks}")
    print(f"[full-size] {name}: tokens {toks} max rel {mx:.2e} mean rel {mn:.2e}", flush=True)
