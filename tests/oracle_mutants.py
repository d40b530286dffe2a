"""Planted mistakes in the oracle, for checking that its pins catch them (test infrastructure only).

Loaded as a pytest plugin (``-p tests.oracle_mutants``) with ORACLE_MUTANT naming one entry of
MUTANTS: before any test module is imported, the named oracle function is replaced by a copy with
one plausible mistake (a dropped term, a wrong sign, index or axis, a wrong rounding).  The pin
suite run that way must fail; tests/test_oracle_mutations.py runs it once per mutant.
"""
from __future__ import annotations

import os

import numpy as np


def _moe():
    from oracle import moe
    return moe


def _codecs():
    from oracle import codecs
    return codecs


def _prefetch():
    from oracle import prefetch
    return prefetch


def silu_sign():
    _moe().silu = lambda z: np.asarray(z, np.float64) / (1.0 + np.exp(np.asarray(z, np.float64)))


def _ffn_parts_with(act):
    m = _moe()

    def parts(X, wg, wu, wd, precision):
        X = np.asarray(X, np.float64)
        G, U = X @ wg.T, X @ wu.T
        A = act(m, G, U)
        codes = scales = None
        if precision == "bf16":
            A = m.bf16_round(A)
        elif precision == "fp8":
            codes, scales = m.quantize_groups(A.astype(np.float32))
            A = m.dequant_groups(codes, scales)
        Y = A @ wd.T
        if precision in ("bf16", "fp8"):
            Y = m.bf16_round(Y)
        return dict(A=A, A_codes=codes, A_scales=scales, Y=Y)
    m.expert_ffn_parts = parts


def swiglu_gate_up_swapped():
    _ffn_parts_with(lambda m, G, U: m.silu(U) * G)


def swiglu_up_dropped():
    _ffn_parts_with(lambda m, G, U: m.silu(G))


def bf16_intermediate_not_rounded():
    m = _moe()

    def parts(X, wg, wu, wd, precision):
        X = np.asarray(X, np.float64)
        A = m.silu(X @ wg.T) * (X @ wu.T)
        codes = scales = None
        if precision == "fp8":
            codes, scales = m.quantize_groups(A.astype(np.float32))
            A = m.dequant_groups(codes, scales)
        Y = A @ wd.T
        if precision in ("bf16", "fp8"):
            Y = m.bf16_round(Y)
        return dict(A=A, A_codes=codes, A_scales=scales, Y=Y)
    m.expert_ffn_parts = parts


def _combine_with(fn):
    m = _moe()

    def combine(y_rows, w, shared_row=None, precision="f32"):
        acc = fn(np.asarray(y_rows, np.float64), np.asarray(w, np.float64), shared_row)
        if precision in ("bf16", "fp8"):
            acc = m.bf16_round(acc)
        return acc
    m.combine = combine


def combine_shared_dropped():
    _combine_with(lambda y, w, s: (w[:, None] * y).sum(0))


def combine_unweighted():
    _combine_with(lambda y, w, s: y.sum(0) + (0 if s is None else np.asarray(s, np.float64)))


def combine_weights_reversed():
    _combine_with(lambda y, w, s: (w[::-1, None] * y).sum(0) + (0 if s is None else np.asarray(s, np.float64)))


def topk_ties_to_higher_index():
    def topk(logits, k):
        l = np.asarray(logits, np.float64)
        E = l.shape[1]
        order = np.lexsort((-np.broadcast_to(np.arange(E), l.shape), -l), axis=1)
        return order[:, :k].astype(np.int32)
    _moe().topk_select = topk


def topk_smallest():
    _moe().topk_select = lambda logits, k: np.argsort(np.asarray(logits, np.float64), axis=1,
                                                      kind="stable")[:, :k].astype(np.int32)


def gate_not_renormalised():
    def gate(logits, idx):
        l = np.asarray(logits, np.float64)
        z = np.exp(l - l.max(axis=1, keepdims=True))
        full = z / z.sum(axis=1, keepdims=True)
        return np.take_along_axis(full, np.asarray(idx, np.int64), axis=1)
    _moe().gate_weights = gate


def router_bias_sign():
    def logits(x, w_router, bias=None):
        l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
        return l if bias is None else l - np.asarray(bias, np.float64)[None, :]
    _moe().router_logits = logits


def router_bias_dropped():
    _moe().router_logits = lambda x, w_router, bias=None: np.asarray(x, np.float64) @ np.asarray(w_router,
                                                                                                 np.float64).T


def _permute_with(order_fn=None, shared_first=False, inverse_is_order=False):
    def permute(idx, E, shared):
        idx = np.asarray(idx, np.int64)
        T, k = idx.shape
        flat = idx.reshape(-1)
        order = order_fn(flat) if order_fn else np.argsort(flat, kind="stable")
        counts = np.bincount(flat, minlength=E)
        offsets = np.zeros(E + shared + 1, np.int64)
        offsets[1:E + 1] = np.cumsum(counts)
        if shared:
            offsets[E + 1] = offsets[E] + T
        src = order // k
        if shared:
            src = np.concatenate([np.arange(T), src] if shared_first else [src, np.arange(T)])
        if inverse_is_order:
            inv = order.copy()
        else:
            inv = np.empty(T * k, np.int64)
            inv[order] = np.arange(T * k)
        return (offsets.astype(np.int32), src.astype(np.int32), inv.reshape(T, k).astype(np.int32),
                counts.astype(np.int64))
    _moe().permute = permute


def permute_reversed_within_expert():
    _permute_with(order_fn=lambda flat: np.lexsort((-np.arange(len(flat)), flat)))


def permute_shared_rows_first():
    _permute_with(shared_first=True)


def permute_inverse_not_inverted():
    _permute_with(inverse_is_order=True)


def _set_codec(name, fn):
    setattr(_codecs(), name, fn)
    setattr(_moe(), name, fn)


def bf16_truncates():
    def trunc(x):
        v = np.asarray(x, np.float64).astype(np.float32)
        bits = v.view(np.uint32) & np.uint32(0xFFFF0000)
        return bits.view(np.float32).astype(np.float64)
    _set_codec("bf16_round", trunc)


def e4m3_ties_away_from_zero():
    c = _codecs()
    pos = c.E4M3_VALUES[:0x7F]

    def enc(x):
        x = np.asarray(x, np.float64)
        a = np.where(np.isnan(x), 0.0, np.minimum(np.abs(x), 448.0))
        hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)
        lo = np.where(pos[hi] > a, hi - 1, hi)
        code = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
        code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
        return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    _set_codec("e4m3_encode", enc)


def e4m3_overflow_to_nan():
    c = _codecs()
    orig = c.e4m3_encode

    def enc(x):
        x = np.asarray(x, np.float64)
        code = orig(x)
        return np.where(np.abs(x) > 448.0, np.uint8(0x7F), code).astype(np.uint8)
    _set_codec("e4m3_encode", enc)


def fp8_scale_uses_fnuz_max():
    def scale(amax32):
        s = (amax32.astype(np.float32) / np.float32(240.0)).astype(np.float32)
        return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)
    _moe()._fp32_scale = scale


def fp8_block_amax_wrong_axes():
    m = _moe()

    def qb(w):
        w32 = np.asarray(w, np.float32)
        o, i = w32.shape
        b = w32.reshape(o // 128, 128, i // 128, 128)
        amax = np.broadcast_to(np.abs(b).max(axis=(0, 1, 3))[None, :], (o // 128, i // 128))   # one per column
        s = m._fp32_scale(amax)
        q = m.e4m3_encode((b / s[:, None, :, None]).astype(np.float32))
        return q.reshape(o, i), s
    m.quantize_blocks = qb


def prefetch_source_major():
    p = _prefetch()

    def plan(sizes, dst_offsets, chunk):
        if chunk <= 0:
            raise ValueError("chunk must be positive")
        out = []
        for s, b in enumerate(sizes):
            for off in range(0, int(b), chunk):
                out.append((s, off, int(dst_offsets[s]) + off, min(chunk, int(b) - off)))
        return out
    p.chunk_plan = plan


def prefetch_last_slice_full():
    p = _prefetch()

    def plan(sizes, dst_offsets, chunk):
        if chunk <= 0:
            raise ValueError("chunk must be positive")
        n = [-(-int(b) // chunk) for b in sizes]
        return [(s, c * chunk, int(dst_offsets[s]) + c * chunk, chunk)
                for c in range(max(n, default=0)) for s in range(len(sizes)) if c < n[s]]
    p.chunk_plan = plan


def fp8_a_not_requantised():
    m = _moe()

    def parts(X, wg, wu, wd, precision):
        X = np.asarray(X, np.float64)
        A = m.silu(X @ wg.T) * (X @ wu.T)
        if precision == "bf16":
            A = m.bf16_round(A)
        Y = A @ wd.T
        if precision in ("bf16", "fp8"):
            Y = m.bf16_round(Y)
        return dict(A=A, A_codes=None, A_scales=None, Y=Y)
    m.expert_ffn_parts = parts


def fp8_scale_divisor_447():
    def scale(amax32):
        s = (amax32.astype(np.float32) / np.float32(447.0)).astype(np.float32)
        return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)
    _moe()._fp32_scale = scale


def fp8_output_not_rounded():
    m = _moe()

    def parts(X, wg, wu, wd, precision):
        X = np.asarray(X, np.float64)
        A = m.silu(X @ wg.T) * (X @ wu.T)
        codes = scales = None
        if precision == "bf16":
            A = m.bf16_round(A)
        elif precision == "fp8":
            codes, scales = m.quantize_groups(A.astype(np.float32))
            A = m.dequant_groups(codes, scales)
        Y = A @ wd.T
        if precision == "bf16":
            Y = m.bf16_round(Y)
        return dict(A=A, A_codes=codes, A_scales=scales, Y=Y)
    m.expert_ffn_parts = parts


def e4m3_subnormals_flushed():
    c = _codecs()
    orig = c.e4m3_encode

    def enc(x):
        x = np.asarray(x, np.float64)
        code = orig(x)
        small = np.abs(x) < 2.0 ** -6                 # below the smallest normal: flushed to a signed zero
        return np.where(small & ~np.isnan(x), (np.signbit(x) * 0x80).astype(np.uint8), code).astype(np.uint8)
    _set_codec("e4m3_encode", enc)


def combine_rounds_each_term():
    m = _moe()

    def combine(y_rows, w, shared_row=None, precision="f32"):
        y = np.asarray(y_rows, np.float64)
        terms = [float(w[j]) * y[j] for j in range(len(w))]
        if precision in ("bf16", "fp8"):
            terms = [m.bf16_round(t) for t in terms]   # a rounding per term instead of one at the end
        acc = np.zeros(y.shape[1:], np.float64)
        for t in terms:
            acc = acc + t
        if shared_row is not None:
            acc = acc + np.asarray(shared_row, np.float64)
        if precision in ("bf16", "fp8"):
            acc = m.bf16_round(acc)
        return acc
    m.combine = combine


def bf16_expert_output_not_rounded():
    m = _moe()
    orig = m.expert_ffn_parts

    def parts(X, wg, wu, wd, precision):
        r = orig(X, wg, wu, wd, precision)
        if precision == "bf16":
            r["Y"] = np.asarray(r["A"], np.float64) @ np.asarray(wd, np.float64).T
        return r
    m.expert_ffn_parts = parts


def fp8_token_groups_64():
    m = _moe()

    def qg(v):
        v32 = np.asarray(v, np.float32)
        n, K = v32.shape
        g = v32.reshape(n, K // 64, 64)                 # 64-wide groups instead of 128
        s = m._fp32_scale(np.abs(g).max(axis=2))
        q = m.e4m3_encode((g / s[:, :, None]).astype(np.float32)).reshape(n, K)
        return q, s[:, ::2]
    m.quantize_groups = qg


MUTANTS = {f.__name__: f for f in [
    silu_sign, swiglu_gate_up_swapped, swiglu_up_dropped, bf16_intermediate_not_rounded,
    combine_shared_dropped, combine_unweighted, combine_weights_reversed,
    topk_ties_to_higher_index, topk_smallest, gate_not_renormalised, router_bias_sign, router_bias_dropped,
    permute_reversed_within_expert, permute_shared_rows_first, permute_inverse_not_inverted,
    bf16_truncates, e4m3_ties_away_from_zero, e4m3_overflow_to_nan, fp8_scale_uses_fnuz_max,
    fp8_block_amax_wrong_axes, fp8_a_not_requantised, fp8_scale_divisor_447, fp8_output_not_rounded,
    prefetch_source_major, prefetch_last_slice_full,
    e4m3_subnormals_flushed, combine_rounds_each_term, bf16_expert_output_not_rounded, fp8_token_groups_64,
]}


def pytest_configure(config):
    name = os.environ.get("ORACLE_MUTANT", "")
    if name:
        MUTANTS[name]()
