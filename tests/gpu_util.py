"""Helpers for the GPU parity tests (imported by test modules; collects no tests)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe

# Relative-error bars (max over elements, mean over elements) of |y - r| / max(|r|, rms(r)).  The fp32,
# bf16 and fp8 maxima are the stated ones.  fp8 states no mean; its mean bar is a tenth of its maximum,
# the same ratio as bf16's, so that a widespread error fails the mean before any single element fails
# the maximum.
TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3), "fp8": dict(max=6e-2, mean=6e-3)}


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


def e4m3_rounding_distance(v_scaled, codes):
    """Distance from each value v (scaled units) to the interval of values that round to the given E4M3
    code (0 where v rounds to it): the interval runs between the midpoints to the neighbouring code
    values, and past 448 for the largest code (saturation)."""
    from oracle import codecs
    vals = np.unique(codecs.E4M3_VALUES[np.isfinite(codecs.E4M3_VALUES)])      # sorted, one zero
    c = codecs.e4m3_decode(codes)
    i = np.searchsorted(vals, c)
    lo = np.where(i > 0, 0.5 * (vals[np.maximum(i - 1, 0)] + c), -np.inf)
    hi = np.where(i < len(vals) - 1, 0.5 * (vals[np.minimum(i + 1, len(vals) - 1)] + c), np.inf)
    v = np.asarray(v_scaled, np.float64)
    return np.maximum(0.0, np.maximum(lo - v, v - hi))


# A re-quantisation flip of an fp8 A code is allowed only where the GPU's code is the rounding of a value
# within FLIP_REL * |v| + FLIP_ABS of the oracle's fp32 value v of A (scaled units, in which the group's
# largest magnitude is 448).  GEMM1 sums each 64-wide fp8 product block in
# the matrix core, whose accumulation of fp8 products is measured here to carry up to about 5e-5 of
# relative error on the largest element of a group (the group scales, amax / 448, of the 16K-token
# fp8 layer differ from the oracle's by up to 4.9e-5), then folds K / 128 block sums with fp32 scale
# products, and SwiGLU uses the hardware exponential.  The windows are about four times that: the
# scale tolerance and the relative window 2e-4, and an absolute window of 1e-4 of the group maximum
# for elements where G and U cancel (the error of a dot product follows the sum of its terms'
# magnitudes, not its result).  With that error about 1.6e-3 of the 16K-token layer's A codes land on
# another code (all within the window); the rate bar is three times that.
FLIP_REL = 2e-4
FLIP_ABS = 448.0 * 1e-4
SCALE_RTOL = 2e-4
FLIP_RATE = 5e-3


def check_fp8_rows(y, a_codes, a_scales, parts, wd, rms, what="", stats=None):
    """fp8 expert rows against the oracle, allowing for re-quantisation flips of A.

    A is re-quantised to E4M3 from an fp32 value that the GPU and the oracle accumulate in
    different orders, so a value within rounding distance of the rounding boundary between two
    codes may land on the neighbouring code.  Rows whose A codes equal the oracle's must meet the
    fp8 tolerance.  A differing code must be the rounding of a value inside the window above around
    the oracle's fp32 A (before its rounding); at most FLIP_RATE of the codes may differ; the scales agree to SCALE_RTOL; and the rows holding flips stay within the
    tolerance plus the flipped codes' effect through the down projection (plus one bf16 rounding).

    y: GPU rows [n, H]; a_codes / a_scales: the GPU's A of the same rows; parts:
    oracle.moe.expert_ffn_parts of the same rows; wd: the prepared down weights [H, I];
    rms: rms of the whole reference the rows belong to; stats: optional dict that accumulates
    codes, flips and the largest flip distance (in units of the allowed window).
    Returns (rows with flips, max rel of the clean rows).
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
    np.testing.assert_allclose(a_scales, parts["A_scales"], rtol=SCALE_RTOL, atol=0, err_msg=f"{what}: A scales")
    worst = 0.0
    if diff.any():
        ri, ci = np.nonzero(diff)
        co, cg = parts["A_codes"][ri, ci], a_codes[ri, ci]
        # the GPU's code must be the rounding of a value within the window around the oracle's fp32 A
        # before rounding (A_pre), in scaled units
        v_scaled = parts["A_pre"][ri, ci] / parts["A_scales"][ri, ci // 128]
        d = e4m3_rounding_distance(v_scaled, cg)
        win = FLIP_REL * np.abs(v_scaled) + FLIP_ABS
        worst = float((d / win).max())
        assert worst <= 1.0, f"{what}: a flipped A code is {worst:.2f} windows from the oracle's A"
        rate = diff.mean()
        assert rate <= FLIP_RATE, f"{what}: {diff.sum()} of {diff.size} A codes differ ({rate:.2e})"
        g = codecs.e4m3_decode(a_codes[flip]).reshape(flip.sum(), -1, 128) * a_scales[flip][:, :, None]
        g = g.reshape(flip.sum(), -1)
        o = parts["A"][flip].reshape(flip.sum(), -1)
        bound = tol * den[flip] + np.abs(g - o) @ np.abs(wd).T * (1 + 1e-6) + np.abs(r[flip]) * 2.0 ** -8
        assert (np.abs(y[flip] - r[flip]) <= bound).all(), f"{what}: a row with flipped A codes is off"
    if stats is not None:
        srel = np.abs(a_scales / parts["A_scales"] - 1.0)
        stats["scale_rel_max"] = max(stats.get("scale_rel_max", 0.0), float(srel.max()))
        stats["codes"] = stats.get("codes", 0) + int(diff.size)
        stats["flips"] = stats.get("flips", 0) + int(diff.sum())
        stats["worst_window"] = max(stats.get("worst_window", 0.0), worst)
    return int(flip.sum()), mx
