"""Helpers for the GPU parity tests (imported by test modules; collects no tests)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe

TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3), "fp8": dict(max=6e-2, mean=6e-2)}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel_err(y, r):
    """max and mean of |y - r| / max(|r|, rms(r)) (elementwise, rms over the whole reference)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    den = np.maximum(np.abs(r), np.sqrt((r ** 2).mean()) + 1e-300)
    e = np.abs(y - r) / den
    return float(e.max()), float(e.mean())


def assert_close(y, r, dtype, what=""):
    mx, mn = rel_err(y, r)
    t = TOL[dtype]
    assert mx <= t["max"] and mn <= t["mean"], f"{what}: max rel {mx:.3e} (tol {t['max']}), mean {mn:.3e}"
    return mx, mn


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


class HostLayer:
    """A small synthetic layer generated on the host (the oracle's inputs)."""

    def __init__(self, cfg: synth.LayerConfig, layer: int = 0, bias=None):
        self.cfg = cfg
        self.x = synth.tokens(cfg, layer)
        self.wr = synth.router_weight(cfg, layer)
        self.bias = synth.router_bias(cfg, layer) if bias is None else bias
        self.experts = [synth.expert_weights(cfg, e, layer) for e in range(cfg.E)]
        self.shared = synth.expert_weights(cfg, cfg.E, layer) if cfg.shared else None

    def oracle(self, routing=None, tokens=None):
        return omoe.moe_layer(self.x, self.wr, self.bias, self.cfg.k, lambda e: self.experts[e],
                              (lambda: self.shared) if self.shared is not None else None,
                              precision=self.cfg.dtype, tokens=tokens, routing=routing)


def upload_layer(h: HostLayer, placement, slots_per_buffer, device="cuda"):
    """ExpertStore + device table + tokens/router for a HostLayer under a placement."""
    from split_weight_expert_amd import ExpertStore
    from split_weight_expert_amd.moe import DTYPES, act_dtype
    cfg = h.cfg
    wd = DTYPES[cfg.dtype]
    adt = act_dtype(wd)
    store = ExpertStore(cfg.H, cfg.I, wd, slots_per_buffer, device=device)
    ws = list(h.experts) + ([h.shared] if h.shared is not None else [])
    for g, (buf, slot) in enumerate(placement):
        wg, wu, wdn = (torch.from_numpy(a).to(device) for a in ws[g])
        if wd != 2:
            wg, wu, wdn = wg.to(adt), wu.to(adt), wdn.to(adt)
        store.load(buf, slot, wg, wu, wdn)
    table = store.table(placement, device)
    x = torch.from_numpy(h.x).to(device).to(adt)
    wr = torch.from_numpy(h.wr).to(device).to(adt)
    b = None if h.bias is None else torch.from_numpy(np.asarray(h.bias, np.float32)).to(device)
    return store, table, x, wr, b
