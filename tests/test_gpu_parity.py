"""Parity of every C-ABI entry point with the CPU oracle on the GPU.

Small shapes that span several tiles and a ragged tail; the bars are
bit-exact for routing indices, permutation and copies, and the stated
tolerances for floating-point outputs (fp32 1e-5 max relative; bf16 2e-2
max / 2e-3 mean; fp8 6e-2 max).
"""
import time

import numpy as np
import pytest
import torch

import synth
from oracle import codecs, moe as omoe
from oracle.prefetch import apply_plan
from synth.configs import shrink
from tests.gpu_util import (TOL, HostLayer, assert_close, check_fp8_rows, ffn_ws_a, need_gpu, rel_err, to_np,
                            upload_layer)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def placement_split(cfg):
    pl = [(0, e) if e < cfg.n_local else (1, e - cfg.n_local) for e in range(cfg.E)]
    if cfg.shared:
        pl.append((0, cfg.n_local))
    return pl, [cfg.n_local + cfg.shared, cfg.E - cfg.n_local]


# --------------------------------------------------------------------------------------- generator

@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_gpu_generator_matches_host_generator(kind):
    from synth import gen
    key = gen.tensor_key(0, 5, 1, 3, 17)
    n = 1_000_003
    out = torch.empty(n, dtype=torch.float32 if kind == "f32" else torch.bfloat16, device=DEV)
    gen.gpu_fill(key, n, 0.37, kind, out.data_ptr(), 0, first=12345)
    torch.cuda.synchronize()
    host = gen.host_fill(key, n, 0.37, kind, first=12345)
    got = out.cpu().numpy() if kind == "f32" else out.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, host)


# --------------------------------------------------------------------------------------- routing

ROUTE_CASES = [
    ("tiny_f32", dict()),
    ("tiny_f32", dict(T=333, E=300, k=7)),          # E not a multiple of 64, ragged T
    ("prefill8k_bf16", dict(T=257, H=1024, E=256, k=8)),
    ("prefill8k_bf16", dict(T=1, H=7168, E=256, k=8)),
    ("decode64_bf16", dict(T=64, H=7168, E=256, k=8)),
    ("tiny_f32", dict(T=5, E=1, k=1)),
    ("tiny_f32", dict(T=9, E=8, k=8)),              # k = E
    ("prefill8k_bf16", dict(T=130, H=512, E=1024, k=32)),   # the largest E and k the router takes
    ("prefill8k_bf16", dict(T=37, H=576, E=200, k=8)),      # 18 K steps over 16 waves, ragged T and E
    ("prefill8k_bf16", dict(T=2100, H=512, E=1000, k=8)),   # over 512 router tiles, ragged T and E
    ("prefill8k_bf16", dict(T=300, H=512, E=200, k=6)),     # the DMA-ring router with ragged T and E
    ("tiny_f32", dict(T=70, E=1024, k=1)),
]


@pytest.mark.parametrize("name,kw", ROUTE_CASES)
def test_route_topk_parity(name, kw):
    from split_weight_expert_amd import api
    cfg = shrink(synth.get_config(name), **kw) if kw else synth.get_config(name)
    x = synth.tokens(cfg)
    wr = synth.router_weight(cfg)
    b = synth.router_bias(cfg)
    adt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    T, E, k = cfg.T, cfg.E, cfg.k
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    api.route_topk(torch.from_numpy(x).to(DEV, adt), torch.from_numpy(wr).to(DEV, adt),
                   None if b is None else torch.from_numpy(b).to(DEV), k, logits, idx, w)
    torch.cuda.synchronize()
    gl, gi, gw = logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
    ref_l = omoe.router_logits(x, wr, b)
    rms = np.sqrt((ref_l ** 2).mean())
    assert np.abs(gl - ref_l).max() <= 1e-5 * rms
    # bit-exact contract: the GPU's selection equals the oracle's selection on the GPU's logits
    np.testing.assert_array_equal(gi, omoe.topk_select(gl, k))
    np.testing.assert_allclose(gw, omoe.gate_weights(gl, gi), rtol=2e-6, atol=1e-7)
    # and the oracle's own routing differs only where its k-th / (k+1)-th margin is below 1e-4 rms
    oi = omoe.topk_select(ref_l, k)
    bad = np.where((gi != oi).any(1))[0]
    for t in bad:
        srt = np.sort(ref_l[t])[::-1]
        assert k < E and srt[k - 1] - srt[k] < 1e-4 * rms


def test_route_all_equal_logits_picks_lowest_indices():
    from split_weight_expert_amd import api
    T, H, E, k = 70, 128, 100, 6
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    wr = torch.zeros(E, H, device=DEV, dtype=torch.bfloat16)
    logits = torch.empty(T, E, device=DEV)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, device=DEV)
    api.route_topk(x, wr, None, k, logits, idx, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
    np.testing.assert_array_equal(w.cpu().numpy(), np.full((T, k), np.float32(1.0 / k)))


# --------------------------------------------------------------------------------------- permute

def run_permute(idx_np, E, shared, x_t, act_dtype):
    from split_weight_expert_amd import api
    T, k = idx_np.shape
    H = x_t.shape[1]
    rows = T * k + shared * T
    fp8 = act_dtype == api.FP8_E4M3
    xp = torch.empty(rows, H, dtype=torch.uint8 if fp8 else x_t.dtype, device=DEV)
    xs = torch.empty(rows, H // 128, dtype=torch.float32, device=DEV) if fp8 else None
    off = torch.empty(E + shared + 1, dtype=torch.int32, device=DEV)
    ps = torch.empty(rows, dtype=torch.int32, device=DEV)
    ip = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(api.workspace_bytes(api.OP_PERMUTE, T, k, E, H, 1, 1, shared), dtype=torch.uint8, device=DEV)
    api.permute(torch.from_numpy(idx_np.astype(np.int32)).to(DEV), E, shared, x_t, act_dtype, xp, xs, off, ps, ip, ws)
    torch.cuda.synchronize()
    return xp, xs, off.cpu().numpy(), ps.cpu().numpy(), ip.cpu().numpy()


# Up to 4096 experts the permutation sorts by chunk histograms (chunks of 1024 entries, or more so that
# there are at most 1024 chunks: 140000 x 8 entries take 973 chunks of 1152, the last one partial); above
# that, by one workgroup per expert (5000).
PERM_CASES = [(64, 8, 2, 0), (1, 1, 1, 1), (1000, 256, 8, 1), (333, 17, 3, 1), (4097, 64, 4, 0), (2, 8, 8, 1),
              (2000, 4096, 8, 0), (300, 5000, 4, 1), (140000, 256, 8, 1)]


@pytest.mark.parametrize("T,E,k,shared", PERM_CASES)
def test_permute_parity_bf16(T, E, k, shared):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(T * 7 + E)
    idx = omoe.topk_select(rng.normal(size=(T, E)), k)
    H = 256
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    xp, _, off, ps, ip = run_permute(idx, E, shared, x, api.BF16)
    r_off, r_ps, r_ip, _ = omoe.permute(idx, E, shared)
    np.testing.assert_array_equal(off, r_off)
    np.testing.assert_array_equal(ps, r_ps)
    np.testing.assert_array_equal(ip, r_ip)
    xb = x.view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(xp.view(torch.int16).cpu().numpy(), xb[r_ps])


def test_permute_skewed_and_empty_experts():
    from split_weight_expert_amd import api
    T, E, k = 3000, 32, 2
    idx = np.zeros((T, k), np.int32)
    idx[:, 0] = 5
    idx[:, 1] = np.where(np.arange(T) % 3 == 0, 9, 31)
    x = torch.randn(T, 128, device=DEV)
    xp, _, off, ps, ip = run_permute(idx, E, 1, x, api.F32)
    r_off, r_ps, r_ip, _ = omoe.permute(idx, E, 1)
    np.testing.assert_array_equal(off, r_off)
    np.testing.assert_array_equal(ps, r_ps)
    np.testing.assert_array_equal(ip, r_ip)
    np.testing.assert_array_equal(xp.cpu().numpy(), x.cpu().numpy()[r_ps])


@pytest.mark.parametrize("T", [1, 64, 515])
def test_permute_fp8_quantisation_is_bit_exact(T):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(T)
    E, k, H = 16, 4, 512
    idx = omoe.topk_select(rng.normal(size=(T, E)), k)
    xf = rng.normal(0, 1, size=(T, H)).astype(np.float32)
    xf[0, :128] = 0.0                                      # an all-zero group
    if T > 3:
        xf[3, 200] = 3000.0                                # a dominant element
    x = torch.from_numpy(xf).to(DEV).to(torch.bfloat16)
    xq, xs, off, ps, ip = run_permute(idx, E, 1, x, api.FP8_E4M3)
    xv = x.float().cpu().numpy()
    q_ref, s_ref = omoe.quantize_groups(xv)
    r_off, r_ps, _, _ = omoe.permute(idx, E, 1)
    np.testing.assert_array_equal(ps, r_ps)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref[r_ps])
    np.testing.assert_array_equal(xs.cpu().numpy(), s_ref[r_ps])


def test_e4m3_device_encoder_on_every_bf16_pattern():
    """The device encoder (through per-token quantisation with unit scales) on all 65536 bf16 inputs."""
    from split_weight_expert_amd import api
    bits = np.arange(2 ** 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    # every row holds 448 at column 0 so that its scale is exactly 1
    n = -(-len(vals) // 127)
    rows = np.zeros((n, 128), np.float32)
    rows[:, 0] = 448.0
    flat = np.zeros(n * 127, np.float32)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(n, 127)
    x = torch.from_numpy(rows).to(DEV).to(torch.bfloat16)
    idx = np.zeros((n, 1), np.int32)
    xq, xs, *_ = run_permute(idx, 1, 0, x, api.FP8_E4M3)
    assert np.all(xs.cpu().numpy() == 1.0)
    np.testing.assert_array_equal(xq.cpu().numpy(), codecs.e4m3_encode(rows))


def test_e4m3_device_encoder_on_every_fp32_pattern_up_to_448():
    """The device's fp32 -> E4M3 encoder on every fp32 value of magnitude <= 448 (normals, subnormals and
    both zeros, both signs: 2 x 1,138,753,537 bit patterns) against the oracle codec.  The values go
    through the block quantiser with unit scales: element 0 of every 128 x 128 block holds 448, so the
    block's scale is 448 / 448 = 1 and every code is the encoder's code of the value itself."""
    from split_weight_expert_amd import api
    from tests import oracle_pool
    top = 0x43E00000                                   # bit pattern of 448.0
    NB, PER = 8192, 128 * 128 - 1                      # blocks per launch, patterns per block
    chunk = NB * PER
    w = torch.empty(NB * 128, 128, dtype=torch.float32, device=DEV)
    q = torch.empty(NB * 128, 128, dtype=torch.uint8, device=DEV)
    s = torch.empty(NB, 1, dtype=torch.float32, device=DEV)
    wv, qv = w.view(NB, 128 * 128), q.view(NB, 128 * 128)
    checked = 0
    t0 = time.time()
    with oracle_pool.e4m3_pool() as ex:
        for sign in (0, 0x80000000):
            for lo in range(0, top + 1, chunk):
                hi = min(top + 1, lo + chunk)
                bits = torch.arange(lo, lo + chunk, dtype=torch.int64, device=DEV)
                bits = torch.where(bits < hi, bits, torch.zeros_like(bits)) | sign      # padding: +-0
                bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32)
                wv[:, 0] = 448.0
                wv[:, 1:] = bits.view(torch.float32).view(NB, PER)
                api.quantize_weight_fp8(w, q, s)
                torch.cuda.synchronize()
                assert bool((s == 1.0).all()) and bool((qv[:, 0] == 0x7E).all())
                got = qv[:, 1:].reshape(-1)[:hi - lo].cpu().numpy()
                ref = oracle_pool.e4m3_codes(lo, hi, sign, ex)
                bad = np.flatnonzero(got != ref)
                assert bad.size == 0, (f"{bad.size} codes differ, first at bit pattern "
                                       f"{(lo + int(bad[0])) | sign:#010x}: device {got[bad[0]]:#04x}, "
                                       f"oracle {ref[bad[0]]:#04x}")
                checked += hi - lo
                print(f"[e4m3] sign {sign >> 31}: patterns {lo:#010x}..{hi - 1:#010x} equal "
                      f"({checked} so far, {time.time() - t0:.0f} s)", flush=True)
    assert checked == 2 * (top + 1)


def test_bf16_device_rounding_on_every_fp32_pattern():
    """The device's fp32 -> bf16 rounding on all 2^32 fp32 bit patterns against the oracle's.  The values
    go through the combine with k = 1, no shared expert, y_perm rows of ones and gate weight w[t] = the
    pattern, so y[t] is the rounding of 0 + w[t] * 1 (the combine's sum starts at +0: -0 gives +0).  The
    oracle's rounding keeps no NaN payload, so a NaN input only has to give a NaN."""
    from split_weight_expert_amd import api
    from tests import oracle_pool
    T, H = 1 << 26, 8
    yp = torch.ones(T, H, dtype=torch.bfloat16, device=DEV)
    inv = torch.arange(T, dtype=torch.int32, device=DEV).view(T, 1)
    w = torch.empty(T, 1, dtype=torch.float32, device=DEV)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    t0 = time.time()
    with oracle_pool.e4m3_pool() as ex:
        for lo in range(0, 1 << 32, T):
            bits = torch.arange(lo, lo + T, dtype=torch.int64, device=DEV)
            bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits).to(torch.int32)
            w.view(-1).copy_(bits.view(torch.float32))
            api.combine(yp, inv, w, 0, y)
            got = y[:, 0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            ref = oracle_pool.bf16_codes(lo, lo + T, ex)
            pat = np.arange(lo, lo + T, dtype=np.uint64).astype(np.uint32)
            nan = (pat & 0x7FFFFFFF) > 0x7F800000
            bad = np.flatnonzero((got != ref) & ~nan)
            assert bad.size == 0, (f"{bad.size} results differ, first at bit pattern {int(pat[bad[0]]):#010x}: "
                                   f"device {got[bad[0]]:#06x}, oracle {ref[bad[0]]:#06x}")
            assert np.all((got[nan] & 0x7FFF) > 0x7F80), "a NaN input gave a non-NaN"
            if (lo // T) % 8 == 7:
                print(f"[bf16] patterns up to {lo + T - 1:#010x} equal ({time.time() - t0:.0f} s)", flush=True)


# --------------------------------------------------------------------------------------- weights fp8

def test_weight_block_quantisation_is_bit_exact():
    from split_weight_expert_amd import api
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(384, 640)).astype(np.float32)
    w[0:128, 128:256] = 0.0
    w[200, 300] = 5.0
    wt = torch.from_numpy(w).to(DEV)
    q = torch.empty(384, 640, dtype=torch.uint8, device=DEV)
    s = torch.empty(3, 5, dtype=torch.float32, device=DEV)
    api.quantize_weight_fp8(wt, q, s)
    torch.cuda.synchronize()
    qr, sr = omoe.quantize_blocks(w)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy(), sr)


# --------------------------------------------------------------------------------------- grouped FFN

FFN_CASES = {
    "f32": ("tiny_f32", dict(T=200)),
    # mean rows per group picks the tile height: ~66 -> 64, ~150 -> 128, ~300 -> 256 (bf16)
    "bf16_bm128": ("prefill8k_bf16", dict(T=300, H=512, I=256, E=4, k=2, n_local=2)),
    "bf16_bm256": ("prefill8k_bf16", dict(T=650, H=768, I=384, E=4, k=2, n_local=2)),
    "bf16": ("prefill8k_bf16", dict(T=200, H=512, I=256, E=8, k=2, n_local=4)),
    "fp8": ("prefill16k_fp8", dict(T=200, H=512, I=256, E=8, k=2, n_local=4)),
    "fp8_bm128": ("prefill16k_fp8", dict(T=300, H=512, I=256, E=4, k=2, n_local=2)),
    # 256-row fp8 tiles when built with DWDP_FP8_BM256 (128-row tiles otherwise)
    "fp8_bm256": ("prefill16k_fp8", dict(T=650, H=768, I=384, E=4, k=2, n_local=2)),
}


def skew_bias(E):
    b = np.zeros(E, np.float32)
    b[0] = 6.0          # most tokens pick expert 0: several m-tiles
    b[E - 1] = -60.0    # nobody picks the last expert: an empty group
    return b


@pytest.mark.parametrize("case", ["f32", "bf16", "fp8", "bf16_bm128", "bf16_bm256", "fp8_bm128", "fp8_bm256"])
def test_grouped_ffn_parity(case):
    from split_weight_expert_amd import MoEBlock
    name, kw = FFN_CASES[case]
    dt = case.split("_")[0]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg, bias=skew_bias(cfg.E))
    pl, slots = placement_split(cfg)
    store, table, x, wr, b = upload_layer(h, pl, slots)
    blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV)
    bb = blk.buffers(cfg.T)
    blk.route(x, wr, b, bb)
    blk.permute(x, bb)
    blk.ffn(table, bb)
    torch.cuda.synchronize()
    off = bb.offsets.cpu().numpy()
    ps = bb.perm_src.cpu().numpy()
    counts = np.diff(off)
    assert counts[0] > 128 and counts[cfg.E - 1] == 0
    assert cfg.rows // (cfg.E + cfg.shared) >= {"bf16_bm128": 96, "bf16_bm256": 192, "fp8_bm128": 96,
                                                 "fp8_bm256": 192}.get(case, 0)
    y_perm = to_np(bb.y_perm).astype(np.float64)
    ws = list(h.experts) + ([h.shared] if h.shared is not None else [])
    ref = np.zeros_like(y_perm)
    X = omoe.prepare_tokens(h.x[ps], cfg.dtype)     # fp8: the oracle's own per-token quantisation
    parts = {}
    for g in range(len(ws)):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            wg, wu, wd = omoe.prepare_weights(*ws[g], cfg.dtype)
            parts[g] = (omoe.expert_ffn_parts(X[r0:r1], wg, wu, wd, cfg.dtype), wd)
            ref[r0:r1] = parts[g][0]["Y"]
    if dt != "fp8":
        assert_close(y_perm, ref, dt, f"grouped ffn {case}")
        return
    # fp8: A is re-quantised from fp32 values accumulated in different orders on the two sides
    codes, scales = ffn_ws_a(bb.ws_ffn, cfg.rows, cfg.I)
    rms = np.sqrt((ref ** 2).mean())
    for g, (pt, wd) in parts.items():
        r0, r1 = off[g], off[g + 1]
        check_fp8_rows(y_perm[r0:r1], codes[r0:r1], scales[r0:r1], pt, wd, rms, f"grouped ffn {case} group {g}")
    assert rel_err(y_perm, ref)[1] <= TOL["fp8"]["mean"]


@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_block_parity(dt):
    from split_weight_expert_amd import MoEBlock
    name, kw = FFN_CASES[dt]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg)
    pl, slots = placement_split(cfg)
    store, table, x, wr, b = upload_layer(h, pl, slots)
    blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV)
    bb = blk.forward(x, wr, b, table)
    torch.cuda.synchronize()
    gl = bb.logits.cpu().numpy().astype(np.float64)
    gi = bb.idx.cpu().numpy()
    np.testing.assert_array_equal(gi, omoe.topk_select(gl, cfg.k))
    # the oracle's layer on the GPU's routing decisions (the routing itself is checked bit-exactly)
    ref = h.oracle(routing=(gl, gi, omoe.gate_weights(gl, gi)))
    np.testing.assert_array_equal(bb.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(bb.inv_perm.cpu().numpy(), ref["inv_perm"])
    assert_close(to_np(bb.y), ref["y"], dt, f"block {dt}")
    # the oracle's own routing agrees wherever its selection margin is not tiny
    own = h.oracle()
    same = (own["idx"] == gi).all(1)
    assert same.mean() > 0.99
    assert_close(to_np(bb.y)[same], own["y"][same], dt, f"block {dt} (oracle routing)")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_placement_invariance_and_determinism(dt):
    from split_weight_expert_amd import MoEBlock
    name, kw = FFN_CASES[dt]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg)
    G = cfg.E + cfg.shared
    rng = np.random.default_rng(11)
    perm = rng.permutation(G)
    placements = {
        "split": placement_split(cfg),
        "all_local": ([(0, g) for g in range(G)], [G, 1]),
        "all_prefetch": ([(1, g) for g in range(G)], [1, G]),
        "scattered": ([(int(perm[g] % 3), int(perm[g] // 3)) for g in range(G)], [-(-G // 3)] * 3),
    }
    outs = {}
    for nm, (pl, slots) in placements.items():
        store, table, x, wr, b = upload_layer(h, pl, slots)
        blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV)
        y1 = blk.forward(x, wr, b, table).y.clone()
        y2 = blk.forward(x, wr, b, table).y.clone()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"{nm}: not deterministic"
        outs[nm] = y1
        del store
    ref = outs["split"].view(torch.int16)
    for nm, y in outs.items():
        assert torch.equal(y.view(torch.int16), ref), f"placement {nm} changed the output"


def test_redundant_placement_two_groups_share_one_record():
    """Two groups pointing at the same record behave like two copies of the same expert."""
    from split_weight_expert_amd import MoEBlock
    name, kw = FFN_CASES["bf16"]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg)
    h.experts[3] = h.experts[2]
    pl, slots = placement_split(cfg)
    store, table, x, wr, b = upload_layer(h, pl, slots)
    pl2 = list(pl)
    pl2[3] = pl[2]                                          # group 3 reads group 2's record
    table2 = store.table(pl2, DEV)
    blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV)
    y1 = blk.forward(x, wr, b, table).y.clone()
    y2 = blk.forward(x, wr, b, table2).y.clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# --------------------------------------------------------------------------------------- combine

@pytest.mark.parametrize("dt,shared", [("f32", 0), ("bf16", 1), ("bf16", 0)])
def test_combine_parity(dt, shared):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(5)
    T, k, H = 300, 8, 1024
    rows = T * k + shared * T
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    yp = torch.randn(rows, H, device=DEV).to(tdt)
    inv = np.stack([rng.permutation(T * k)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    y = torch.empty(T, H, dtype=tdt, device=DEV)
    api.combine(yp, torch.from_numpy(inv).to(DEV), torch.from_numpy(w).to(DEV), shared, y)
    torch.cuda.synchronize()
    ypn = to_np(yp)
    ref = np.stack([omoe.combine(ypn[inv[t]], w[t], ypn[T * k + t] if shared else None, dt) for t in range(T)])
    assert_close(to_np(y), ref, dt, "combine")


# --------------------------------------------------------------------------------------- prefetch

@pytest.mark.parametrize("engine", [0, 1, 2])
def test_prefetch_copies_every_byte(engine):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(engine)
    # an empty source, short last slices and an odd byte count (the copy kernel's vector tail and byte tail)
    sizes = [1_000_000, 3_333_344, 0, 2_097_152, 777_777]
    chunk = 262_144
    srcs_np = [rng.integers(0, 256, size=n, dtype=np.uint8) for n in sizes]
    srcs = [torch.from_numpy(a).to(DEV) if len(a) else torch.empty(16, dtype=torch.uint8, device=DEV)
            for a in srcs_np]
    offs = [0, 1_000_000, 4_333_344, 4_333_344, 6_430_496]
    total = offs[-1] + sizes[-1] + 64
    dst = torch.full((total,), 7, dtype=torch.uint8, device=DEV)
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    done = torch.cuda.Event()
    api.prefetch_chunks(dst.data_ptr(), [(s.data_ptr(), o, n) for s, o, n in zip(srcs, offs, sizes)], chunk,
                        engine=engine, max_workgroups=5, copy_stream=cs, done_event=done)
    torch.cuda.current_stream().wait_event(done)
    got = dst.cpu().numpy()
    ref = apply_plan(np.full(total, 7, np.uint8), srcs_np, offs, chunk)
    np.testing.assert_array_equal(got, ref)


def test_prefetch_waits_for_the_last_reader():
    """The copy must not start before the event it is told to wait on (the last reader of the slots)."""
    from split_weight_expert_amd import api
    n = 64 << 20
    src = torch.full((n,), 3, dtype=torch.uint8, device=DEV)
    dst = torch.zeros(n, dtype=torch.uint8, device=DEV)
    reader = torch.cuda.Stream()
    cs = torch.cuda.Stream()
    snap = torch.empty(n, dtype=torch.uint8, device=DEV)
    gate = torch.cuda.Event()
    done = torch.cuda.Event()
    reader.wait_stream(torch.cuda.current_stream())
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(reader):
        torch.cuda._sleep(50_000_000)                       # keep the reader busy for a while
        snap.copy_(dst)                                     # the reader's view of the slots
        gate.record(reader)
    api.prefetch_chunks(dst.data_ptr(), [(src.data_ptr(), 0, n)], 4 << 20, engine=1, copy_stream=cs,
                        wait_event=gate, done_event=done)
    torch.cuda.synchronize()
    assert int(snap.max()) == 0                             # the reader saw the old contents
    assert int(dst.min()) == 3                              # and the copy then completed


# --------------------------------------------------------------------------------------- weight layout

@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_pack_weights_matches_the_documented_layout(dt):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(21)
    N, K = 96, 384
    if dt == "bf16":
        w = rng.integers(0, 2 ** 16, size=(N, K), dtype=np.uint16)
        wt = torch.from_numpy(w.view(np.int16)).to(DEV).view(torch.bfloat16)
        out = torch.empty_like(wt)
        api.pack_weights(wt, out, api.BF16)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, 8)
        q = np.arange(N * K // 8)
        frag, l, per = q // 64, q % 64, K // 16
        rows = (frag // per) * 32 + l % 32
        cols = (frag % per) * 16 + (l // 32) * 8
        exp = np.stack([w[rows, cols + e] for e in range(8)], axis=1)
    else:
        w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        wt = torch.from_numpy(w).to(DEV)
        out = torch.empty_like(wt)
        api.pack_weights(wt, out, api.FP8_E4M3)
        got = out.cpu().numpy().reshape(-1, 16)
        q = np.arange(N * K // 16)
        frag, h, l, per = q // 128, (q // 64) % 2, q % 64, K // 64
        rows = (frag // per) * 32 + l % 32
        cols = (frag % per) * 64 + (l // 32) * 32 + h * 16
        exp = np.stack([w[rows, cols + e] for e in range(16)], axis=1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, exp)


# --------------------------------------------------------------------------------------- token-row GEMM1

@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_token_rows_equal_permuted_rows(dt):
    """GEMM1 reading token rows through perm_src gives bitwise the x_perm path's A, y_perm and y."""
    from split_weight_expert_amd import MoEBlock, api
    name, kw = FFN_CASES[dt]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg, bias=skew_bias(cfg.E))
    pl, slots = placement_split(cfg)
    store, table, x, wr, b = upload_layer(h, pl, slots)
    out = {}
    for gather in (True, False):
        blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV, gather=gather)
        bb = blk.buffers(cfg.T)
        blk.route(x, wr, b, bb)
        blk.permute(x, bb)
        if gather:
            # the plain entry point (both stages in one call)
            api.moe_grouped_ffn(table, cfg.E + cfg.shared, bb.offsets, bb.x_perm, bb.x_perm_scale, cfg.H, cfg.I,
                                blk.w_dtype, bb.y_perm, bb.ws_ffn)
        else:
            assert bb.x_perm is None
            blk.ffn(table, bb)
        blk.combine(bb)
        torch.cuda.synchronize()
        ea = 4 if dt == "f32" else 2 if dt == "bf16" else 1
        out[gather] = dict(perm_src=bb.perm_src.clone(), offsets=bb.offsets.clone(), y_perm=bb.y_perm.clone(),
                           y=bb.y.clone(), A=bb.ws_ffn[:cfg.rows * cfg.I * ea].clone())
    for key in out[True]:
        assert torch.equal(out[True][key], out[False][key]), key


@pytest.mark.parametrize("H", [1024, 7168, 8960])   # 8, 56 and 70 groups: one and two batches of loads
def test_token_quantiser_is_bit_exact(H):
    from split_weight_expert_amd import api
    cfg = shrink(synth.get_config("prefill16k_fp8"), T=300, H=H)
    x = synth.tokens(cfg)
    x[5] = 0.0                                    # an all-zero token: scale 1
    xt = torch.from_numpy(x).to(DEV, torch.bfloat16)
    q = torch.empty(cfg.T, cfg.H, dtype=torch.uint8, device=DEV)
    s = torch.empty(cfg.T, cfg.H // 128, dtype=torch.float32, device=DEV)
    api.quantize_tokens_fp8(xt, q, s)
    torch.cuda.synchronize()
    qr, sr = omoe.quantize_groups(xt.float().cpu().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy(), sr)


def test_per_token_kernels_walk_more_tokens_than_their_grid():
    """The per-token kernels launch at most 2^20 workgroups and walk the rest: token quantiser and combine
    (one workgroup per token) at 2^20 + 37 tokens, top-k (four tokens per workgroup) at 2^22 + 11."""
    from split_weight_expert_amd import api
    rng = np.random.default_rng(41)
    T, H = (1 << 20) + 37, 128
    x = torch.from_numpy(rng.normal(size=(T, H)).astype(np.float32)).to(DEV, torch.bfloat16)
    q = torch.empty(T, H, dtype=torch.uint8, device=DEV)
    s = torch.empty(T, 1, dtype=torch.float32, device=DEV)
    api.quantize_tokens_fp8(x, q, s)
    torch.cuda.synchronize()
    qr, sr = omoe.quantize_groups(x.float().cpu().numpy())
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy(), sr)
    # combine, k = 2 with a shared row, H = 8
    k, Hc = 2, 8
    yp = torch.from_numpy(rng.normal(size=(T * k + T, Hc)).astype(np.float32)).to(DEV, torch.bfloat16)
    ip_np = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w_np = rng.random((T, k)).astype(np.float32)
    y = torch.empty(T, Hc, dtype=torch.bfloat16, device=DEV)
    api.combine(yp, torch.from_numpy(ip_np).to(DEV), torch.from_numpy(w_np).to(DEV), 1, y)
    torch.cuda.synchronize()
    ypn = to_np(yp)
    acc = np.zeros((T, Hc))
    for j in range(k):                           # the oracle's combine, vectorised over tokens
        acc = acc + w_np[:, j:j + 1].astype(np.float64) * ypn[ip_np[:, j]]
    ref = codecs.bf16_round(acc + ypn[T * k:])
    assert_close(to_np(y), ref, "bf16", "combine over 2^20 + 37 tokens")
    # top-k on f32 logits of 2^22 + 11 tokens, E = 8, k = 3
    T2, Hr, E, kk = (1 << 22) + 11, 16, 8, 3
    xr = torch.from_numpy(rng.normal(size=(T2, Hr)).astype(np.float32)).to(DEV)
    wr = torch.from_numpy(rng.normal(size=(E, Hr)).astype(np.float32)).to(DEV)
    logits = torch.empty(T2, E, dtype=torch.float32, device=DEV)
    idx = torch.empty(T2, kk, dtype=torch.int32, device=DEV)
    wt = torch.empty(T2, kk, dtype=torch.float32, device=DEV)
    api.route_topk(xr, wr, None, kk, logits, idx, wt)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    np.testing.assert_array_equal(idx.cpu().numpy(), omoe.topk_select(gl, kk))


@pytest.mark.parametrize("shared", [0, 1])
def test_permute_without_gather_gives_the_same_indices(shared):
    from split_weight_expert_amd import api
    T, k, E, H = 517, 4, 37, 256
    rng = np.random.default_rng(3)
    idx_np = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    rows = T * k + shared * T
    res = []
    for with_rows in (True, False):
        idx = torch.from_numpy(idx_np).to(DEV)
        xp = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV) if with_rows else None
        off = torch.empty(E + shared + 1, dtype=torch.int32, device=DEV)
        ps = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
        ip = torch.empty(T, k, dtype=torch.int32, device=DEV)
        ws = torch.empty(api.workspace_bytes(api.OP_PERMUTE, T, k, E, H, 1, api.BF16, shared), dtype=torch.uint8,
                         device=DEV)
        api.permute(idx, E, shared, x, api.BF16, xp, None, off, ps, ip, ws)
        torch.cuda.synchronize()
        res.append((off.cpu().numpy(), ps.cpu().numpy(), ip.cpu().numpy()))
    o, p, i = omoe.permute(idx_np, E, shared)[:3]
    for r in res:
        np.testing.assert_array_equal(r[0], o)
        np.testing.assert_array_equal(r[1], p)
        np.testing.assert_array_equal(r[2], i)


def test_grouped_ffn_with_more_groups_than_one_schedule_pass():
    """1500 routed experts + a shared one: the tile schedule scans and sorts groups in several passes."""
    from split_weight_expert_amd import ExpertStore, api
    from split_weight_expert_amd.moe import DTYPES
    cfg = shrink(synth.get_config("prefill8k_bf16"), T=400, H=256, I=128, E=1500, k=2, n_local=1500)
    rng = np.random.default_rng(11)
    idx_np = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    idx_np[:40] = [3, 7]                                  # one group with 40+ rows
    x = synth.tokens(cfg)
    xt = torch.from_numpy(x).to(DEV, torch.bfloat16)
    G = cfg.E + 1
    store = ExpertStore(cfg.H, cfg.I, DTYPES["bf16"], [G], device=DEV)
    used = sorted(set(idx_np.ravel().tolist()) | {cfg.E})
    weights = {}
    for e in used:
        weights[e] = synth.expert_weights(cfg, e)
        store.load(0, e, *(torch.from_numpy(a).to(DEV, torch.bfloat16) for a in weights[e]))
    table = store.table([(0, g) for g in range(G)], DEV)
    rows = cfg.T * (cfg.k + 1)
    off = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    ps = torch.empty(rows, dtype=torch.int32, device=DEV)
    ip = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=DEV)
    wsp = torch.empty(api.workspace_bytes(api.OP_PERMUTE, cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, api.BF16, 1),
                      dtype=torch.uint8, device=DEV)
    api.permute(torch.from_numpy(idx_np).to(DEV), cfg.E, 1, xt, api.BF16, None, None, off, ps, ip, wsp)
    y_perm = torch.empty(rows, cfg.H, dtype=torch.bfloat16, device=DEV)
    wsf = torch.empty(api.workspace_bytes(api.OP_GROUPED_FFN, cfg.T, cfg.k, cfg.E, cfg.H, cfg.I, api.BF16, 1),
                      dtype=torch.uint8, device=DEV)
    api.moe_grouped_ffn_tokens(0, table, G, off, ps, xt, None, cfg.H, cfg.I, api.BF16, y_perm, wsf)
    torch.cuda.synchronize()
    o, p, _, counts = omoe.permute(idx_np, cfg.E, 1)
    np.testing.assert_array_equal(off.cpu().numpy(), o)
    np.testing.assert_array_equal(ps.cpu().numpy(), p)
    y = to_np(y_perm).astype(np.float64)
    ref = np.zeros_like(y)
    for g in used:
        r0, r1 = o[g], o[g + 1]
        if r1 > r0:
            ref[r0:r1] = omoe.expert_ffn(omoe.prepare_tokens(x[p[r0:r1]], "bf16"),
                                         *omoe.prepare_weights(*weights[g], "bf16"), "bf16")
    assert_close(y, ref, "bf16", "grouped ffn, 1501 groups")


def test_empty_batch_is_a_no_op_for_every_step():
    """T = 0: every entry point returns OK and touches nothing."""
    from split_weight_expert_amd import api
    H, I, E, k = 256, 128, 8, 2
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(E, H, dtype=torch.bfloat16, device=DEV)
    logits = torch.empty(0, E, device=DEV)
    idx = torch.empty(0, k, dtype=torch.int32, device=DEV)
    w = torch.empty(0, k, device=DEV)
    api.route_topk(x, wr, None, k, logits, idx, w)
    off = torch.full((E + 2,), -5, dtype=torch.int32, device=DEV)
    ps = torch.empty(0, dtype=torch.int32, device=DEV)
    ws = torch.empty(4096, dtype=torch.uint8, device=DEV)
    api.permute(idx, E, 1, x, api.BF16, None, None, off, ps, idx, ws)
    api.quantize_tokens_fp8(x, torch.empty(0, H, dtype=torch.uint8, device=DEV),
                            torch.empty(0, H // 128, device=DEV))
    y = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    api.combine(torch.empty(0, H, dtype=torch.bfloat16, device=DEV), idx, w, 1, y)
    torch.cuda.synchronize()
    assert (off.cpu() == -5).all()         # T = 0 returns before anything is written


# --------------------------------------------------------------------------------------- dropped entries

@pytest.mark.parametrize("E", [16, 5000])
def test_permute_and_combine_drop_out_of_range_indices(E):
    """topk_idx entries outside [0, E) are dropped (include/dwdp.h, dwdp_permute): counted in no expert,
    inv_perm -1, skipped by the combine; offsets[E] stays T*k and the rows closing the last routed group
    read token 0 (defined, never read back).  E = 16 sorts by chunk histograms, E = 5000 by expert."""
    from split_weight_expert_amd import api
    T, k, H, S = 300, 4, 256, 1
    rng = np.random.default_rng(17)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    bad = [(0, 1, -1), (5, 0, E), (17, 3, E + 5), (120, 2, -7), (299, 0, 1 << 20)]
    for t, j, v in bad:
        idx[t, j] = v
    valid = (idx >= 0) & (idx < E)
    x = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    _, _, off, ps, ip = run_permute(idx, E, S, x, api.BF16)
    # the expected permutation of the valid entries: experts ascending, then flattened t*k+j
    flat = np.flatnonzero(valid.ravel())
    order = flat[np.argsort(idx.ravel()[flat], kind="stable")]
    counts = np.bincount(idx.ravel()[flat], minlength=E)
    n_valid, D = len(order), T * k - len(order)
    exp_off = np.concatenate([[0], np.cumsum(counts)[:-1], [T * k, T * k + T]])
    np.testing.assert_array_equal(off, exp_off)
    exp_ip = np.full(T * k, -1, np.int64)
    exp_ip[order] = np.arange(n_valid)
    np.testing.assert_array_equal(ip.ravel(), exp_ip)
    np.testing.assert_array_equal(ps[:n_valid], order // k)
    np.testing.assert_array_equal(ps[n_valid:T * k], np.zeros(D, np.int32))       # the dropped rows: token 0
    np.testing.assert_array_equal(ps[T * k:], np.arange(T))
    # the combine skips the dropped slots
    rows = T * k + S * T
    yp = torch.randn(rows, H, device=DEV).to(torch.bfloat16)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    api.combine(yp, torch.from_numpy(ip).to(DEV), torch.from_numpy(w).to(DEV), S, y)
    torch.cuda.synchronize()
    ypn = to_np(yp)
    ref = np.stack([omoe.combine(ypn[ip[t][valid[t]]], w[t][valid[t]], ypn[T * k + t], "bf16") for t in range(T)])
    assert_close(to_np(y), ref, "bf16", "combine with dropped slots")   # fp32 sums vs fp64: one rounding apart


# --------------------------------------------------------------------------------------- deep K, every tail

# Group sizes chosen so that the last m-tile of the groups holds every row count the kernels have a
# variant for.  With a mean of 192 or more rows per group bf16 runs 256-row tiles: tails of 20, 50, 80,
# 120, 144, 180, 204, 250 and 256 rows (1..8 active 32-row blocks, spread over the two 128-row halves);
# fp8 runs 128-row tiles there too unless the library is built with DWDP_FP8_BM256, which gives it
# 256-row tiles.  The fp8_bm128 case (mean rows per group 96..191) runs 128-row fp8 tiles: tails of 20,
# 50, 80, 120 and 128 rows.  An empty group is included.  K = 2048 (GEMM1) and 1024 (GEMM2) are deep
# enough for the steady-state loops of every DMA ring (bf16 and 256-row fp8 tiles step 64 bytes of K:
# 64 and 32 steps for bf16 and 32 and 16 for fp8, against NS + P = 8 and 7; 128-row fp8 tiles step
# 128 bytes: 16 and 8 steps against NS + P - 1 = 4).
TAIL_CASES = {
    "bf16": dict(H=2048, I=1024, sizes=[276, 306, 336, 376, 400, 436, 460, 506, 512, 0, 20]),
    "fp8": dict(H=2048, I=1024, sizes=[276, 306, 336, 376, 400, 436, 460, 506, 512, 0, 20]),
    "fp8_bm128": dict(H=2048, I=1024, sizes=[148, 178, 208, 248, 20, 36, 40, 70, 100, 0, 60, 90]),
}


def normal_expert(rng, H, I):
    """(Wg, Wu, Wd) float32 ~ N(0, 1/fan_in) from numpy's normal generator (true normal tails)."""
    return (rng.normal(0, H ** -0.5, size=(I, H)).astype(np.float32),
            rng.normal(0, H ** -0.5, size=(I, H)).astype(np.float32),
            rng.normal(0, I ** -0.5, size=(H, I)).astype(np.float32))


@pytest.mark.parametrize("case", ["bf16", "fp8", "fp8_bm128"])
def test_grouped_ffn_every_tail_variant_deep_k(case):
    """Every y_perm row of a grouped FFN whose groups end on every tile-tail variant, at K large enough
    for the steady-state DMA ring loops, against the oracle's expert FFN; inputs from numpy's normal
    generator (unbounded tails, which set the fp8 group maxima)."""
    from split_weight_expert_amd import ExpertStore, api
    from split_weight_expert_amd.moe import DTYPES
    c = TAIL_CASES[case]
    dt = case.split("_")[0]
    H, I, sizes = c["H"], c["I"], c["sizes"]
    E, k, S = len(sizes), 1, 1
    T = int(sum(sizes))
    rng = np.random.default_rng({"bf16": 123, "fp8": 321, "fp8_bm128": 231}[case])
    idx = np.repeat(np.arange(E), sizes).astype(np.int32)[rng.permutation(T)].reshape(T, 1)
    x = rng.normal(0, 1, size=(T, H)).astype(np.float32)
    x[7, 5] = 9.0                                              # an outlier sets one group's scale
    experts = [normal_expert(rng, H, I) for _ in range(E + S)]
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()     # tokens enter as bf16 (fp8 too)
    if dt == "bf16":                                           # bf16 layers hold bf16 weights; fp8 quantises fp32
        experts = [tuple(torch.from_numpy(w).to(torch.bfloat16).float().numpy() for w in ex) for ex in experts]
    wd = DTYPES[dt]
    G = E + S
    store = ExpertStore(H, I, wd, [(G + 1) // 2, G // 2], device=DEV)
    pl = [(g % 2, g // 2) for g in range(G)]                   # groups alternate between two buffers
    for g, (b_, s_) in enumerate(pl):
        ws_ = [torch.from_numpy(w).to(DEV) for w in experts[g]]
        if dt == "bf16":
            ws_ = [w.to(torch.bfloat16) for w in ws_]
        store.load(b_, s_, *ws_)
    table = store.table(pl, DEV)
    xt = torch.from_numpy(x).to(DEV, torch.bfloat16)
    rows = T * (k + S)
    off = torch.empty(G + 1, dtype=torch.int32, device=DEV)
    ps = torch.empty(rows, dtype=torch.int32, device=DEV)
    ip = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wsp = torch.empty(api.workspace_bytes(api.OP_PERMUTE, T, k, E, H, I, wd, S), dtype=torch.uint8, device=DEV)
    api.permute(torch.from_numpy(idx).to(DEV), E, S, xt, api.BF16, None, None, off, ps, ip, wsp)
    xq = xs = None
    if dt == "fp8":
        xq = torch.empty(T, H, dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, H // 128, dtype=torch.float32, device=DEV)
        api.quantize_tokens_fp8(xt, xq, xs)
    y_perm = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    wsf = torch.empty(api.workspace_bytes(api.OP_GROUPED_FFN, T, k, E, H, I, wd, S), dtype=torch.uint8, device=DEV)
    api.moe_grouped_ffn_tokens(0, table, G, off, ps, xq if dt == "fp8" else xt, xs, H, I, wd, y_perm, wsf)
    torch.cuda.synchronize()
    o, p, _, counts = omoe.permute(idx, E, S)
    np.testing.assert_array_equal(off.cpu().numpy(), o)
    np.testing.assert_array_equal(ps.cpu().numpy(), p)
    np.testing.assert_array_equal(counts, sizes)
    y = to_np(y_perm).astype(np.float64)
    X = omoe.prepare_tokens(x[p], dt)
    if dt == "bf16":
        ref = np.zeros_like(y)
        for g in range(G):
            r0, r1 = o[g], o[g + 1]
            if r1 > r0:
                ref[r0:r1] = omoe.expert_ffn(X[r0:r1], *omoe.prepare_weights(*experts[g], dt), dt)
        mx, mn = assert_close(y, ref, dt, "grouped ffn, every tail, deep K")
        print(f"[tails bf16] rows {rows} max rel {mx:.2e} mean rel {mn:.2e}", flush=True)
        return
    codes, scales = ffn_ws_a(wsf, rows, I)
    parts = {}
    for g in range(G):
        r0, r1 = o[g], o[g + 1]
        if r1 > r0:
            wts = omoe.prepare_weights(*experts[g], dt)
            parts[g] = (omoe.expert_ffn_parts(X[r0:r1], *wts, dt), wts[2])
    ref = np.concatenate([parts[g][0]["Y"] for g in sorted(parts)])
    rms = np.sqrt((ref ** 2).mean())
    stats = {}
    clean_mx, flipped = 0.0, 0
    for g, (pt, w2) in parts.items():
        r0, r1 = o[g], o[g + 1]
        # rows whose A codes equal the oracle's meet the fp8 maximum; rows with re-quantisation flips are
        # bounded by the flips' effect (check_fp8_rows)
        nf, cm = check_fp8_rows(y[r0:r1], codes[r0:r1], scales[r0:r1], pt, w2, rms, f"{case} tails group {g}", stats)
        clean_mx, flipped = max(clean_mx, cm), flipped + nf
    mx, mn = rel_err(y, ref)
    assert mn <= TOL["fp8"]["mean"], f"mean rel {mn:.2e}"
    print(f"[tails {case}] rows {rows} max rel {mx:.2e} (rows without flips {clean_mx:.2e}; {flipped} rows with "
          f"flips) mean rel {mn:.2e}; A codes {stats['codes']}, "
          f"flips {stats['flips']} ({stats['flips'] / stats['codes']:.2e}), worst flip "
          f"{stats['worst_window']:.3f} windows, scales within {stats['scale_rel_max']:.1e}", flush=True)
