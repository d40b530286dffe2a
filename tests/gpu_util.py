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


def ffn_ws_a(ws: torch.Tensor, rows: int, I: int, sel=None):
    """A's E4M3 codes [rows, I] and scales [rows, I/128] as the grouped FFN leaves them in its workspace
    (layout documented with dwdp_moe_grouped_ffn in include/dwdp.h); only rows `sel` if given."""
    n = rows * I
    off = (n + 255) // 256 * 256
    codes = ws[:n].view(rows, I)
    scales = ws[off:off + rows * (I // 128) * 4].view(torch.float32).view(rows, I // 128)
    if sel is not None:
        idx = torch.as_tensor(np.asarray(sel, np.int64), device=ws.device)
        codes, scales = codes[idx], scales[idx]
    return codes.cpu().numpy(), scales.cpu().numpy()


def check_fp8_rows(y, a_codes, a_scales, parts, wd, rms, what=""):
    """fp8 expert rows against the oracle, allowing for re-quantisation flips of A.

    A is re-quantised to E4M3 from an fp32 value that the GPU and the oracle accumulate in
    different orders, so a value within rounding distance of a midpoint between two codes may
    land on the neighbouring code (and a group's amax, with it the scale, differs by the fp32
    accumulation error of GEMM1, up to about 1e-4 relative).  Rows whose A codes equal the
    oracle's must meet the fp8 tolerance.  At most 1 in 100 codes may differ, each by one code
    step plus 1e-4 of its group's amax, and the rows holding them must stay within the
    tolerance plus the flipped codes' effect through the down projection (plus one bf16
    rounding).

    y: GPU rows [n, H]; a_codes / a_scales: the GPU's A of the same rows; parts:
    oracle.moe.expert_ffn_parts of the same rows; wd: the prepared down weights [H, I];
    rms: rms of the whole reference the rows belong to.  Returns (rows with flips, max rel of
    the clean rows).
    """
    from oracle import codecs
    r = parts["Y"]
    y = np.asarray(y, np.float64)
    den = np.maximum(np.abs(r), rms)
    tol = TOL["fp8"]["max"]
    diff = a_codes != parts["A_codes"]
    flip = diff.any(1)
    clean = ~flip
    mx = float((np.abs(y - r) / den)[clean].max()) if clean.any() else 0.0
    assert mx <= tol, f"{what}: clean rows max rel {mx:.3e} (tol {tol})"
    assert diff.mean() <= 1e-2, f"{what}: {diff.sum()} of {diff.size} A codes differ"
    # the scales follow each group's amax, which carries the fp32 accumulation error of GEMM1
    np.testing.assert_allclose(a_scales, parts["A_scales"], rtol=2e-4, atol=0, err_msg=f"{what}: A scales")
    if flip.any():
        g = codecs.e4m3_decode(a_codes[flip]).reshape(flip.sum(), -1, 128) * a_scales[flip][:, :, None]
        o = parts["A"][flip].reshape(flip.sum(), -1, 128)
        g = g.reshape(flip.sum(), -1)
        o = o.reshape(flip.sum(), -1)
        # neighbouring codes: one E4M3 step (1/8 of the larger magnitude, or one subnormal step) plus
        # the fp32 accumulation error of A, taken as 1e-4 of its group's amax (= 448 * scale)
        sc = np.repeat(np.maximum(a_scales[flip], parts["A_scales"][flip]), 128, axis=1)
        step = np.maximum(np.abs(g), np.abs(o)) / 8.0 + sc * 2.0 ** -9 + 1e-4 * 448.0 * sc
        assert (np.abs(g - o) <= step * (1 + 1e-6)).all(), f"{what}: a flipped A code is not a neighbour"
        bound = tol * den[flip] + np.abs(g - o) @ np.abs(wd).T * (1 + 1e-6) + np.abs(r[flip]) * 2.0 ** -8
        assert (np.abs(y[flip] - r[flip]) <= bound).all(), f"{what}: a row with flipped A codes is off"
    return int(flip.sum()), mx
