"""Pins of the oracle's MoE layer: closed forms, brute force, library routines and invariants.

Each test checks the oracle against something other than itself, so that a
dropped term, a wrong sign or index, or a transposed operand fails one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import moe
from synth.configs import shrink


# ----------------------------------------------------------------------------------------------
# helpers written independently of the oracle

def brute_topk(row, k):
    """Repeatedly take the largest remaining logit, lower index first on ties (pure Python)."""
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


def torch_ffn(x, wg, wu, wd):
    """FFN through torch's CPU linear/silu in float64 (a library routine, not the oracle's code)."""
    f = torch.nn.functional
    X = torch.from_numpy(np.asarray(x, np.float64))
    g = f.linear(X, torch.from_numpy(np.asarray(wg, np.float64)))
    u = f.linear(X, torch.from_numpy(np.asarray(wu, np.float64)))
    return f.linear(f.silu(g) * u, torch.from_numpy(np.asarray(wd, np.float64))).numpy()


def dense_masked_layer(x, wr, b, k, experts, shared):
    """Evaluate every expert on every token and mask with the gate (brute force)."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = len(experts)
    logits = x @ np.asarray(wr, np.float64).T + (0 if b is None else np.asarray(b, np.float64))
    full = scipy.special.softmax(logits, axis=1)
    mask = np.zeros((T, E))
    for t in range(T):
        chosen = brute_topk(list(logits[t]), k)
        mask[t, chosen] = full[t, chosen] / full[t, chosen].sum()
    y = np.zeros_like(x)
    for e in range(E):
        y += mask[:, e:e + 1] * torch_ffn(x, *experts[e])
    if shared is not None:
        y += torch_ffn(x, *shared)
    return y


def tiny_layer(cfg, E=None, k=None, shared=None):
    x = synth.tokens(cfg)
    wr = synth.router_weight(cfg)
    b = synth.router_bias(cfg)
    ex = [synth.expert_weights(cfg, e) for e in range(cfg.E)]
    return x, wr, b, ex


TINY = synth.get_config("tiny_f32")


# ----------------------------------------------------------------------------------------------
# gate

def test_zero_router_gives_first_k_experts_with_equal_weights():
    T, H, E, k = 5, 16, 8, 3
    x = np.random.default_rng(0).normal(size=(T, H))
    l, idx, w = moe.route(x, np.zeros((E, H)), np.zeros(E), k)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k), (T, 1)))
    assert np.all(w == 1.0 / k) or np.allclose(w, 1.0 / k, rtol=0, atol=1e-16)


def test_topk_matches_brute_force_with_many_ties():
    rng = np.random.default_rng(1)
    logits = rng.integers(-3, 4, size=(300, 12)).astype(np.float64)   # many exact ties
    for k in (1, 2, 5, 12):
        got = moe.topk_select(logits, k)
        for t in range(len(logits)):
            assert list(got[t]) == brute_topk(list(logits[t]), k)


def test_topk_treats_signed_zeros_as_equal():
    logits = np.array([[0.0, -0.0, 0.0, -1.0]])
    np.testing.assert_array_equal(moe.topk_select(logits, 3), [[0, 1, 2]])


def test_gate_weights_closed_form():
    logits = np.array([[0.0, math.log(3.0), -50.0]])
    idx = moe.topk_select(logits, 2)
    np.testing.assert_array_equal(idx, [[1, 0]])
    np.testing.assert_allclose(moe.gate_weights(logits, idx), [[0.75, 0.25]], rtol=0, atol=1e-15)


def test_gate_equals_full_softmax_renormalised():
    rng = np.random.default_rng(2)
    logits = rng.normal(0, 3, size=(200, 64))
    for k in (1, 4, 8):
        idx = moe.topk_select(logits, k)
        w = moe.gate_weights(logits, idx)
        full = scipy.special.softmax(logits, axis=1)
        sel = np.take_along_axis(full, idx, 1)
        np.testing.assert_allclose(w, sel / sel.sum(1, keepdims=True), rtol=1e-14, atol=0)
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
        assert np.all(np.diff(w, axis=1) <= 0)      # slots ordered by weight descending


def test_router_logits_transposition_and_bias():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(3, 5))
    wr = rng.normal(size=(4, 5))
    b = rng.normal(size=4)
    l = moe.router_logits(x, wr, b)
    for t, e in itertools.product(range(3), range(4)):
        assert abs(l[t, e] - (sum(x[t, h] * wr[e, h] for h in range(5)) + b[e])) < 1e-12


# ----------------------------------------------------------------------------------------------
# permutation

def brute_permutation(idx, E):
    """O(E*T*k) triple loop: walk experts in order, and inside each the assignments in order."""
    T, k = idx.shape
    src, inv = [], np.full((T, k), -1)
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    inv[t, j] = len(src)
                    src.append(t)
    return np.array(src), inv


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 4, 2), (33, 8, 3), (64, 16, 16)])
def test_permutation_matches_triple_loop(T, E, k):
    rng = np.random.default_rng(T * 100 + E)
    logits = rng.normal(size=(T, E))
    idx = moe.topk_select(logits, k)
    offsets, src, inv, counts = moe.permute(idx, E, shared=0)
    bsrc, binv = brute_permutation(idx, E)
    np.testing.assert_array_equal(src, bsrc)
    np.testing.assert_array_equal(inv, binv)
    assert counts.sum() == T * k and offsets[-1] == T * k
    np.testing.assert_array_equal(np.diff(offsets), counts)


def test_permutation_invariants_with_shared_group():
    rng = np.random.default_rng(5)
    T, E, k = 50, 8, 2
    idx = moe.topk_select(rng.normal(size=(T, E)), k)
    offsets, src, inv, counts = moe.permute(idx, E, shared=1)
    R = T * k
    assert len(offsets) == E + 2 and offsets[E] == R and offsets[E + 1] == R + T
    np.testing.assert_array_equal(src[R:], np.arange(T))
    for t in range(T):
        for j in range(k):
            assert src[inv[t, j]] == t
            e = idx[t, j]
            assert offsets[e] <= inv[t, j] < offsets[e + 1]
    flat_pos = np.empty(R, np.int64)
    flat_pos[inv.reshape(-1)] = np.arange(R)            # flattened (t*k+j) of each permuted row
    for e in range(E):
        seg = flat_pos[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)                 # stable: increasing inside an expert
    x = rng.normal(size=(T, 4))
    xp = x[src]
    for t in range(T):
        for j in range(k):
            np.testing.assert_array_equal(xp[inv[t, j]], x[t])   # permute then unpermute is identity


def test_permutation_with_empty_and_full_experts():
    T, E, k = 10, 5, 1
    idx = np.full((T, k), 3, np.int32)                   # every token to expert 3
    offsets, src, inv, counts = moe.permute(idx, E, shared=0)
    np.testing.assert_array_equal(offsets, [0, 0, 0, 0, T, T])
    np.testing.assert_array_equal(src, np.arange(T))


# ----------------------------------------------------------------------------------------------
# FFN and the layer

def test_silu_matches_logistic():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(moe.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert moe.silu(0.0) == 0.0


def test_single_expert_reduces_to_plain_ffn():
    rng = np.random.default_rng(6)
    T, H, I = 9, 12, 5                                   # H != I catches transposed operands
    x = rng.normal(size=(T, H))
    wg, wu, wd = rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))
    out = moe.moe_layer(x, rng.normal(size=(1, H)), None, 1, lambda e: (wg, wu, wd))
    np.testing.assert_array_equal(out["w"], np.ones((T, 1)))
    np.testing.assert_allclose(out["y"], torch_ffn(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def test_dense_masked_brute_force_equals_sparse_oracle_tiny_workload():
    x, wr, b, ex = tiny_layer(TINY)
    out = moe.moe_layer(x, wr, b, TINY.k, lambda e: ex[e])
    ref = dense_masked_layer(x, wr, b, TINY.k, ex, None)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("T,H,I,E,k", [(13, 24, 16, 5, 2), (20, 32, 8, 6, 6), (4, 16, 16, 3, 1)])
def test_dense_masked_brute_force_random_shapes_with_shared(T, H, I, E, k):
    rng = np.random.default_rng(T + H + E)
    x = rng.normal(size=(T, H))
    wr, b = rng.normal(size=(E, H)), rng.normal(size=E)
    ex = [(rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I))) for _ in range(E)]
    sh = (rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I)))
    out = moe.moe_layer(x, wr, b, k, lambda e: ex[e], lambda: sh)
    ref = dense_masked_layer(x, wr, b, k, ex, sh)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_token_subset_equals_full_layer_rows():
    x, wr, b, ex = tiny_layer(TINY)
    full = moe.moe_layer(x, wr, b, TINY.k, lambda e: ex[e])
    sub = [3, 0, 63, 17]
    part = moe.moe_layer(x, wr, b, TINY.k, lambda e: ex[e], tokens=sub)
    np.testing.assert_allclose(part["y"], full["y"][sub], rtol=1e-12, atol=1e-13)


def test_zero_down_projection_leaves_shared_expert_only():
    rng = np.random.default_rng(7)
    T, H, I, E, k = 11, 16, 8, 4, 2
    x = rng.normal(size=(T, H))
    ex = [(rng.normal(size=(I, H)), rng.normal(size=(I, H)), np.zeros((H, I))) for _ in range(E)]
    sh = (rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I)))
    out = moe.moe_layer(x, rng.normal(size=(E, H)), None, k, lambda e: ex[e], lambda: sh)
    np.testing.assert_allclose(out["y"], torch_ffn(x, *sh), rtol=1e-12, atol=1e-12)


def test_duplicated_experts_give_the_same_output():
    rng = np.random.default_rng(8)
    T, H, I, E, k = 16, 16, 8, 4, 1
    x = rng.normal(size=(T, H))
    w = (rng.normal(size=(I, H)), rng.normal(size=(I, H)), rng.normal(size=(H, I)))
    a = moe.moe_layer(x, rng.normal(size=(E, H)), None, k, lambda e: w)
    b = moe.moe_layer(x, rng.normal(size=(E, H)), None, k, lambda e: w)   # other routing
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["y"], torch_ffn(x, *w), rtol=1e-12, atol=1e-12)


def test_bf16_policy_rounds_outputs_to_bf16_values():
    cfg = shrink(synth.get_config("decode64_bf16"), T=8, H=256, I=128, E=8, k=2)
    x, wr, b, ex = tiny_layer(cfg)
    sh = synth.expert_weights(cfg, cfg.E)
    out = moe.moe_layer(x, wr, b, cfg.k, lambda e: ex[e], lambda: sh, precision="bf16")
    y = out["y"]
    np.testing.assert_array_equal(y, y.astype(np.float32).astype(np.float64))
    assert np.all((y.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)   # bf16 numbers
    ref = moe.moe_layer(x, wr, b, cfg.k, lambda e: ex[e], lambda: sh, precision="f32")["y"]
    rel = np.abs(y - ref) / np.maximum(np.abs(ref), np.sqrt((ref ** 2).mean()))
    assert rel.max() < 2e-2 and rel.mean() < 2e-3                      # rounding error only


def test_bf16_policy_rounds_the_intermediate_before_the_down_projection():
    """Rounding point of the bf16 policy: A = silu(X Wg^T) * (X Wu^T) is rounded to bf16 (torch's own
    conversion) before it meets Wd, and Y is the bf16 rounding of that A times Wd^T."""
    cfg = shrink(synth.get_config("decode64_bf16"), T=8, H=256, I=128, E=8, k=2)
    x, wr, b, ex = tiny_layer(cfg)
    wg, wu, wd = moe.prepare_weights(*ex[3], "bf16")
    X = moe.prepare_tokens(x, "bf16")
    parts = moe.expert_ffn_parts(X, wg, wu, wd, "bf16")
    f = torch.nn.functional
    Xt = torch.from_numpy(np.asarray(X, np.float64))
    a = f.silu(f.linear(Xt, torch.from_numpy(wg))) * f.linear(Xt, torch.from_numpy(wu))
    a_bf16 = a.to(torch.bfloat16).to(torch.float64)
    np.testing.assert_array_equal(parts["A"], a_bf16.numpy())
    y = f.linear(a_bf16, torch.from_numpy(wd)).to(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.abs(y) * 2.0 ** -7
    assert np.all(np.abs(parts["Y"] - y) <= ulp)          # equal up to one bf16 step (fp64 sum order)
    assert np.mean(parts["Y"] == y) > 0.99


# ----------------------------------------------------------------------------------------------
# fp8 quantisation

def test_group_quantisation_properties():
    rng = np.random.default_rng(9)
    v = rng.normal(0, 2, size=(6, 512)).astype(np.float32)
    v[2, 128:256] = 0.0                                   # an all-zero group
    v[3, 0] = 1000.0                                      # a dominant element
    q, s = moe.quantize_groups(v)
    assert q.shape == v.shape and s.shape == (6, 4)
    assert s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    g = np.abs(v).reshape(6, 4, 128)
    for r in range(6):
        for c in range(4):
            if g[r, c].max() > 0:
                j = int(np.argmax(g[r, c]))
                assert q[r, c * 128 + j] & 0x7F == 0x7E    # the group maximum maps to +-448
    deq = moe.dequant_groups(q, s)
    bound = 2.0**-4 * np.abs(v) + np.repeat(s, 128, axis=1) * 2.0**-10 * 1.0001
    assert np.all(np.abs(deq - v) <= bound)


def test_block_quantisation_is_local_to_each_block():
    rng = np.random.default_rng(10)
    w = rng.normal(0, 0.05, size=(256, 384)).astype(np.float32)
    q0, s0 = moe.quantize_blocks(w)
    assert s0.shape == (2, 3)
    w2 = w.copy()
    w2[130, 300] = 7.0                                    # inside block (1, 2)
    q1, s1 = moe.quantize_blocks(w2)
    changed = s1 != s0
    assert changed[1, 2] and changed.sum() == 1
    diff = q1 != q0
    assert diff[128:, 256:].any() and not diff[:128].any() and not diff[:, :256].any()
    assert q1[130, 300] == 0x7E
    deq = moe.dequant_blocks(q0, s0)
    sc = np.repeat(np.repeat(s0, 128, 0), 128, 1)
    assert np.all(np.abs(deq - w) <= 2.0**-4 * np.abs(w) + sc * 2.0**-10 * 1.0001)


def test_fp8_policy_dense_equals_sparse():
    cfg = shrink(synth.get_config("prefill16k_fp8"), T=12, H=256, I=128, E=4, k=2)
    x, wr, b, ex = tiny_layer(cfg)
    out = moe.moe_layer(x, wr, b, cfg.k, lambda e: ex[e], precision="fp8")
    # brute force: every expert on every token with the same value policy, masked by the gate
    xq = moe.prepare_tokens(x, "fp8")
    y = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = out["idx"][t, j]
            Y = moe.expert_ffn(xq, *moe.prepare_weights(*ex[e], "fp8"), "fp8")
            y[t] += out["w"][t, j] * Y[t]
    np.testing.assert_allclose(out["y"], moe.bf16_round(y), rtol=0, atol=1e-12 + 2**-7 * np.abs(y).max())


def test_fp8_expert_against_torch_float8():
    """Tokens through one fp8 expert with H = I = 128, written out with torch's float8_e4m3fn.

    At H = I = 128 every weight matrix is a single 128x128 block and every token row (and every
    row of the intermediate A) a single 128-wide group, so each scale is one amax / 448 (fp32).
    The expert is spelled out from that definition: tokens and weights quantised and dequantised
    with torch's E4M3 conversion, G and U in float64, A = silu(G) * U re-quantised per row before
    the down projection, Y rounded to bf16 with torch's conversion.  This pins the re-quantisation
    of A, the 448 in the scale and the bf16 rounding of the expert output (reading 10 of the fp8
    policy; the pages' own format is NVFP4, DWDP paper summary Section 5.1).
    """
    rng = np.random.default_rng(21)
    x = rng.normal(0, 1, size=(8, 128)).astype(np.float32)
    x[3] *= 40.0                                          # a token with large values
    wg, wu, wd = (rng.normal(0, 128 ** -0.5, size=(128, 128)).astype(np.float32) for _ in range(3))

    def q(v, rows):
        """Quantise v per row (rows=True) or as one block; returns (dequantised fp64, codes, scales)."""
        v = torch.from_numpy(np.ascontiguousarray(v, np.float32))
        amax = v.abs().amax(dim=1, keepdim=True) if rows else v.abs().max().reshape(1, 1)
        s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)          # fp32 division
        c = (v / s).to(torch.float8_e4m3fn)
        return c.to(torch.float64) * s.to(torch.float64), c.view(torch.uint8).numpy(), s.numpy()

    xd = q(x, True)[0]
    wgd, wud, wdd = (q(w, False)[0] for w in (wg, wu, wd))
    f = torch.nn.functional
    a = f.silu(xd @ wgd.T) * (xd @ wud.T)
    ad, a_codes, a_scales = q(a.to(torch.float32).numpy(), True)
    y = (ad @ wdd.T).to(torch.bfloat16).to(torch.float64).numpy()

    parts = moe.expert_ffn_parts(moe.prepare_tokens(x, "fp8"), *moe.prepare_weights(wg, wu, wd, "fp8"), "fp8")
    assert parts["A_codes"] is not None
    np.testing.assert_array_equal(parts["A_codes"], a_codes)
    np.testing.assert_array_equal(parts["A_scales"], a_scales[:, :1].reshape(-1, 1))
    np.testing.assert_array_equal(parts["A"], ad.numpy())
    ulp = np.abs(y) * 2.0 ** -7
    assert np.all(np.abs(parts["Y"] - y) <= ulp)          # equal up to one bf16 step (fp64 sum order)
    assert np.mean(parts["Y"] == y) > 0.99


def test_combine_rounds_once_after_the_sum():
    """The combine sums the weighted rows and rounds once (bf16 policy): worked by hand.
    w = [2^-2 + 3*2^-11, 2^-1 + 2^-10] on two rows of ones.  The exact sum is 0.75244140625, above the
    midpoint 0.751953125 between the bf16 neighbours 0.75 and 0.75390625, so it rounds to 0.75390625.
    Rounding each term first (0.25146484375 -> 0.251953125, 0.5009765625 -> 0.5) would give 0.751953125,
    a tie that rounds to the even 0.75."""
    y = moe.combine(np.array([[1.0], [1.0]]), np.array([0.25146484375, 0.5009765625], np.float32), None, "bf16")
    assert y.tolist() == [0.75390625]
