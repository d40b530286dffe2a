"""The MoE layer, plainly (oracle; test infrastructure only).

DWDP keeps attention replicated and splits the MoE experts across ranks; a
rank fetches the experts it lacks and then runs an ordinary MoE layer on its
own batch (DWDP paper summary, §2 Methodology Overview).  The grouped GEMM
reads split buffers instead of a merged copy, which changes no result (§4.2).
So this module is the textbook layer; the pages give no formula for it, and
the readings taken where they are silent are:

  gate      logits l = W_r x + b; the k experts with the largest logits are
            chosen (equal logits: lower expert index first; slots ordered by
            logit descending); their weights are the softmax over the chosen k,
            which equals the full softmax renormalised over them.
  expert    FFN_e(x) = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + e^-z),
            weights stored [out, in].
  shared    one always-on expert, weight 1, added after the routed sum.
  layer     y_t = sum_j w_tj FFN_{S_tj}(x_t) + FFN_shared(x_t).
  permute   rows ordered by expert, and inside an expert by the flattened
            (token * k + slot) index; the shared expert's rows (all tokens in
            order) follow the routed rows.

Precision policies (rounding points of the GPU's data types, applied here as
data policy with this module's own codecs):
  "f32"   everything in fp64, no rounding points.
  "bf16"  A = silu(G)*U rounded to bf16; expert outputs rounded to bf16; the
          combined output rounded to bf16 once.
  "fp8"   tokens quantised per token in 1x128 groups and weights in 128x128
          blocks to E4M3 with fp32 scales (scale = amax / 448, or 1 when amax
          is 0, codes = E4M3(v / scale), both divisions in fp32); A quantised
          like the tokens (from its fp32 value); expert outputs and the
          combined output rounded to bf16.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round, e4m3_decode, e4m3_encode

GROUP = 128          # fp8 activation group width and weight block edge


# ----------------------------------------------------------------------------------------------
# gate

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * w_router[e, h] + bias[e], in fp64."""
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def topk_select(logits, k: int) -> np.ndarray:
    """Per row, the k largest logits' expert indices, ordered by (logit desc, index asc)."""
    order = np.argsort(-np.asarray(logits, np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_weights(logits, idx) -> np.ndarray:
    """Softmax over the chosen k logits of each row (fp64)."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(idx, np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int):
    l = router_logits(x, w_router, bias)
    idx = topk_select(l, k)
    return l, idx, gate_weights(l, idx)


# ----------------------------------------------------------------------------------------------
# permutation

def permute(idx, E: int, shared: int):
    """Counting-sort permutation of the (token, slot) assignments by expert.

    Returns offsets [E+shared+1] (row ranges of each group), perm_src [T*k + shared*T]
    (source token of each permuted row), inv_perm [T, k] (permuted row of each
    assignment) and counts [E].
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + shared + 1, np.int64)
    offsets[1:E + 1] = np.cumsum(counts)
    if shared:
        offsets[E + 1] = offsets[E] + T
    src = order // k
    if shared:
        src = np.concatenate([src, np.arange(T)])
    inv = np.empty(T * k, np.int64)
    inv[order] = np.arange(T * k)
    return (offsets.astype(np.int32), src.astype(np.int32), inv.reshape(T, k).astype(np.int32),
            counts.astype(np.int64))


# ----------------------------------------------------------------------------------------------
# fp8 quantisation

def _fp32_scale(amax32: np.ndarray) -> np.ndarray:
    s = (amax32.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    return np.where(amax32 == 0, np.float32(1.0), s).astype(np.float32)


def quantize_groups(v):
    """Per row, per group of 128 columns: scale = amax/448 (fp32), codes = E4M3(v/scale) (fp32).

    v [n, K] is taken to fp32 first.  Returns (codes uint8 [n, K], scales float32 [n, K/128]).
    """
    v32 = np.asarray(v, np.float32)
    n, K = v32.shape
    g = v32.reshape(n, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    s = _fp32_scale(amax)
    q = e4m3_encode((g / s[:, :, None]).astype(np.float32))
    return q.reshape(n, K), s


def quantize_blocks(w):
    """Per 128x128 block of w [out, in]: scale = amax/448 (fp32), codes = E4M3(w/scale) (fp32).

    Returns (codes uint8 [out, in], scales float32 [out/128, in/128]).
    """
    w32 = np.asarray(w, np.float32)
    o, i = w32.shape
    b = w32.reshape(o // GROUP, GROUP, i // GROUP, GROUP)
    amax = np.abs(b).max(axis=(1, 3))
    s = _fp32_scale(amax)
    q = e4m3_encode((b / s[:, None, :, None]).astype(np.float32))
    return q.reshape(o, i), s


def dequant_groups(q, s) -> np.ndarray:
    n, K = q.shape
    return (e4m3_decode(q).reshape(n, K // GROUP, GROUP) * np.asarray(s, np.float64)[:, :, None]).reshape(n, K)


def dequant_blocks(q, s) -> np.ndarray:
    o, i = q.shape
    v = e4m3_decode(q).reshape(o // GROUP, GROUP, i // GROUP, GROUP)
    return (v * np.asarray(s, np.float64)[:, None, :, None]).reshape(o, i)


# ----------------------------------------------------------------------------------------------
# expert FFN and combine

def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def prepare_weights(wg, wu, wd, precision: str):
    """The weight values the FFN multiplies by: as given, or their fp8 block dequantisation."""
    if precision == "fp8":
        return tuple(dequant_blocks(*quantize_blocks(w)) for w in (wg, wu, wd))
    return tuple(np.asarray(w, np.float64) for w in (wg, wu, wd))


def prepare_tokens(x, precision: str) -> np.ndarray:
    """The token values the FFN sees: as given, or their per-token fp8 group dequantisation."""
    if precision == "fp8":
        return dequant_groups(*quantize_groups(x))
    return np.asarray(x, np.float64)


def expert_ffn_parts(X, wg, wu, wd, precision: str) -> dict:
    """The expert FFN with its intermediate: Y = W_d (silu(W_g X) * (W_u X)) for the rows of X.

    X and the weights are the prepared values (see prepare_tokens / prepare_weights).  Returns
    A (the intermediate as the down projection consumes it, after the policy's rounding point),
    A_pre, A_codes and A_scales (fp8 only: the fp32 value of A that is quantised, its E4M3 codes
    and its group scales) and Y.
    """
    X = np.asarray(X, np.float64)
    G = X @ wg.T
    U = X @ wu.T
    A = silu(G) * U
    pre = codes = scales = None
    if precision == "bf16":
        A = bf16_round(A)
    elif precision == "fp8":
        pre = A.astype(np.float32)
        codes, scales = quantize_groups(pre)
        A = dequant_groups(codes, scales)
    Y = A @ wd.T
    if precision in ("bf16", "fp8"):
        Y = bf16_round(Y)
    return dict(A=A, A_pre=pre, A_codes=codes, A_scales=scales, Y=Y)


def expert_ffn(X, wg, wu, wd, precision: str) -> np.ndarray:
    """Y = W_d (silu(W_g X) * (W_u X)) for the rows of X, with the policy's rounding points.

    X and the weights are the prepared values (see prepare_tokens / prepare_weights).
    """
    return expert_ffn_parts(X, wg, wu, wd, precision)["Y"]


def combine(y_rows, w, shared_row=None, precision: str = "f32") -> np.ndarray:
    """y = sum_j w[j] * y_rows[j] (+ shared_row), summed in slot order, rounded once per policy."""
    acc = np.zeros(np.asarray(y_rows).shape[1:], np.float64)
    for j in range(len(w)):
        acc = acc + float(w[j]) * np.asarray(y_rows[j], np.float64)
    if shared_row is not None:
        acc = acc + np.asarray(shared_row, np.float64)
    if precision in ("bf16", "fp8"):
        acc = bf16_round(acc)
    return acc


# ----------------------------------------------------------------------------------------------
# the layer

def moe_layer(x, w_router, bias, k: int, experts, shared_expert=None, precision: str = "f32",
              tokens=None, routing=None):
    """One MoE layer on tokens x [T, H].

    experts(e) -> (Wg [I,H], Wu [I,H], Wd [H,I]) generated weights of routed expert e;
    shared_expert() -> the same for the shared expert, or None for no shared expert.
    tokens: optional token indices whose outputs are computed (routing and permutation
    always cover all T tokens); routing: optional (logits, idx, w) to use instead of the
    oracle's own gate.  Experts are visited one at a time, so a full layer's weights are
    never held at once.
    Returns a dict with logits, idx, w, offsets, perm_src, inv_perm, counts, tokens, y.
    """
    x = np.asarray(x)
    T, H = x.shape
    E = np.asarray(w_router).shape[0]
    if routing is None:
        logits, idx, w = route(x, w_router, bias, k)
    else:
        logits, idx, w = routing
    S = 1 if shared_expert is not None else 0
    offsets, perm_src, inv_perm, counts = permute(idx, E, S)
    sel = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    pos_of = {int(t): i for i, t in enumerate(sel)}
    R = T * k

    # permuted rows needed by the selected tokens, grouped by expert
    need = {}
    for t in sel:
        for j in range(k):
            p = int(inv_perm[t, j])
            need.setdefault(int(idx[t, j]), []).append(p)
    y_perm = {}
    for e in sorted(need):
        rows = sorted(need[e])
        wg, wu, wd = prepare_weights(*experts(e), precision)
        X = prepare_tokens(x[perm_src[rows]], precision)
        Y = expert_ffn(X, wg, wu, wd, precision)
        for r, p in enumerate(rows):
            y_perm[p] = Y[r]
    y_shared = None
    if S:
        wg, wu, wd = prepare_weights(*shared_expert(), precision)
        y_shared = expert_ffn(prepare_tokens(x[sel], precision), wg, wu, wd, precision)

    y = np.zeros((len(sel), H), np.float64)
    for i, t in enumerate(sel):
        rows = np.stack([y_perm[int(inv_perm[t, j])] for j in range(k)])
        y[i] = combine(rows, w[t], None if y_shared is None else y_shared[i], precision)
    return dict(logits=logits, idx=idx, w=w, offsets=offsets, perm_src=perm_src, inv_perm=inv_perm,
                counts=counts, tokens=sel, y=y, R=R, pos_of=pos_of)
