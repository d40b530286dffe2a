"""The library's diagnostics on the GPU: the operand-stream probe, and the expert GEMM's tile trace.

The tile trace is compiled in only with -DDWDP_TILE_TRACE=1; its test loads such a build
(split_weight_expert_amd/lib/trace/libdwdp.so, made by split_weight_expert_amd/build.py --out) and
checks that the traced launch ran every tile of the schedule exactly once and that the trace build
computes the default build's results bit for bit.
"""
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRACE_LIB = os.path.join(ROOT, "split_weight_expert_amd", "lib", "trace", "libdwdp.so")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_operand_stream_probe_runs_every_configuration():
    from split_weight_expert_amd import api
    span, grid = 64 << 10, 4
    buf = torch.ones(grid * span, dtype=torch.uint8, device=DEV)
    for in_flight in range(1, 6):
        for cpol in (0, 2):
            api.diag_operand_stream(buf, span, span, 2, grid, in_flight, cpol)
            api.diag_operand_stream(buf, span, 0, 3, grid, in_flight, cpol)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        api.diag_operand_stream(buf, span, span, 1, grid + 1)        # would read past the tensor


def test_lds_read_probe_reports_a_plausible_rate():
    from split_weight_expert_amd import api
    for waves in (4, 8, 16):
        bpc, ghz = api.diag_lds_read(4, waves, 200)
        assert 0.5 < ghz < 3.0 and 16 < bpc < 4096, (waves, bpc, ghz)


def _problem(dt, counts, H, I, seed):
    from split_weight_expert_amd import ExpertStore, api
    from split_weight_expert_amd.moe import DTYPES
    rng = np.random.default_rng(seed)
    G = len(counts)
    rows = int(sum(counts))
    store = ExpertStore(H, I, DTYPES[dt], [G], device=DEV)
    for g in range(G):
        w = [torch.from_numpy(rng.standard_normal(s).astype(np.float32) / np.sqrt(s[1])).to(DEV)
             for s in ((I, H), (I, H), (H, I))]
        store.load(0, g, *w)
    table = store.table([(0, g) for g in range(G)], DEV)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
    x = torch.from_numpy(rng.standard_normal((rows, H)).astype(np.float32)).to(DEV, torch.bfloat16)
    if dt == "fp8":
        xq = torch.empty(rows, H, dtype=torch.uint8, device=DEV)
        xs = torch.empty(rows, H // 128, dtype=torch.float32, device=DEV)
        api.quantize_tokens_fp8(x, xq, xs)
        x, x_scale, wcode = xq, xs, api.FP8_E4M3
    else:
        x_scale, wcode = None, api.BF16
    ws = torch.empty(api.workspace_bytes(api.OP_GROUPED_FFN, rows, 1, G, H, I, wcode, 0), dtype=torch.uint8,
                     device=DEV)
    return store, table, offsets, x, x_scale, wcode, ws, rows


# 128-row tiles dealt over the XCDs; and 32-row tiles drawn from the ticket counter (a few rows per group,
# as in decode, one group of several m-tiles among them)
COUNTS = {"dealt": [0, 3, 40, 300, 700, 64, 1, 257, 33],
          "tickets": [2, 0, 5, 1, 7, 3, 100, 4, 0, 6, 1, 2, 33, 5, 3, 1, 0, 8, 2, 64]}


@pytest.mark.parametrize("dt,mode", [("bf16", "dealt"), ("fp8", "dealt"), ("bf16", "tickets"), ("fp8", "tickets")])
def test_tile_trace_covers_every_tile_once_and_changes_no_result(dt, mode):
    if not os.path.exists(TRACE_LIB):
        pytest.skip("no tile-trace build (DWDP_EXTRA_FLAGS=-DDWDP_TILE_TRACE=1 split_weight_expert_amd/build.py "
                    "--out split_weight_expert_amd/lib/trace/libdwdp.so)")
    from split_weight_expert_amd import _lib, api
    H, I = 512, 256
    counts = COUNTS[mode]
    G = len(counts)
    store, table, offsets, x, x_scale, wcode, ws, rows = _problem(dt, counts, H, I, seed=5)
    y_default = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    api.moe_grouped_ffn_stage(0, table, G, offsets, x, x_scale, H, I, wcode, y_default, ws)
    torch.cuda.synchronize()

    saved = _lib._lib
    _lib._lib = None
    try:
        _lib.load(TRACE_LIB)
        assert "tile-trace=1" in api.version()
        y_trace = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
        traces = {}
        for stage in (1, 2, 2):     # stage 2 twice: the second launch finds its ticket counter reset
            api.diag_tile_trace_clear()
            api.moe_grouped_ffn_stage(stage, table, G, offsets, x, x_scale, H, I, wcode, y_trace, ws)
            torch.cuda.synchronize()
            tr = api.diag_tile_trace_read(4096)
            traces[stage] = tr[tr["t_end"] > 0]
    finally:
        _lib._lib = saved
    assert torch.equal(y_trace, y_default), "the tile-trace build changed the results"
    # tile heights: 32 rows where the tiles draw tickets, 128 where they are dealt
    assert (traces[1]["rows"].max() <= 32) == (mode == "tickets")

    off = np.concatenate([[0], np.cumsum(counts)])
    for stage, n_tiles in ((1, I // 128), (2, H // 256)):
        tr = traces[stage]
        assert (tr["t_end"] >= tr["t_start"]).all()
        assert ((tr["xcd"] >= 0) & (tr["xcd"] < 8)).all()
        assert len(np.unique(tr["order"])) == len(tr), "a schedule position ran twice"
        for g in range(G):
            mine = tr[tr["group"] == g]
            if counts[g] == 0:
                assert len(mine) == 0
                continue
            for nt in range(n_tiles):
                cov = np.zeros(counts[g], np.int32)
                for r in mine[mine["n_tile"] == nt]:
                    lo = r["first_row"] - off[g]
                    assert 0 <= lo and lo + r["rows"] <= counts[g] and r["rows"] > 0
                    cov[lo:lo + r["rows"]] += 1
                assert (cov == 1).all(), f"stage {stage} group {g} n-tile {nt}: rows covered {np.unique(cov)}"
            assert set(mine["n_tile"].tolist()) == set(range(n_tiles))
            assert (mine["group_m_tiles"] == len(np.unique(mine["first_row"]))).all()


def _coverage(tr, counts, n_tiles):
    """Every (group, n-tile) of the schedule ran: its tiles' rows cover the group's rows exactly once."""
    off = np.concatenate([[0], np.cumsum(counts)])
    assert len(np.unique(tr["order"])) == len(tr), "a schedule position ran twice"
    seen = np.zeros((len(counts), n_tiles), np.int64)
    for g in np.unique(tr["group"]):
        mine = tr[tr["group"] == g]
        for nt in range(n_tiles):
            sel = mine[mine["n_tile"] == nt]
            cov = np.zeros(counts[g], np.int32)
            for r in sel:
                lo = r["first_row"] - off[g]
                assert 0 <= lo and lo + r["rows"] <= counts[g] and r["rows"] > 0
                cov[lo:lo + r["rows"]] += 1
            assert (cov == 1).all(), f"group {g} n-tile {nt}: rows covered {np.unique(cov)}"
            seen[g, nt] = len(sel)
        assert (mine["group_m_tiles"] == len(np.unique(mine["first_row"]))).all()
    assert (tr["t_end"] >= tr["t_start"]).all()
    assert ((seen > 0) == (np.asarray(counts)[:, None] > 0)).all(), "a non-empty group missed an n-tile"


# Full-size tile schedules (H = 7168, I = 2048, 256 routed experts + 1 shared): every group's table entry
# points at one shared expert record, so only the row counts -- all the schedule depends on -- are real.
FULL_COUNTS = {
    # 8K bf16-like: skewed counts summing to 65536 routed rows, some empty, + 8192 shared rows
    "prefill8k_bf16": ("bf16", 11),
    # 16K fp8-like: near-balanced counts (131072 routed rows) + 16384 shared
    "prefill16k_fp8": ("fp8", 12),
    # decode-like: 512 routed rows over 256 experts (32-row ticket tiles) + 64 shared
    "decode64_bf16": ("bf16", 13),
}


def _full_counts(name, seed):
    rng = np.random.default_rng(seed)
    E = 256
    if name == "prefill8k_bf16":
        w = rng.pareto(1.2, E) + 0.02
        w[rng.choice(E, 9, replace=False)] = 0
        counts = rng.multinomial(65536, w / w.sum())
        return np.concatenate([counts, [8192]])
    if name == "prefill16k_fp8":
        counts = rng.multinomial(131072, np.full(E, 1.0 / E))
        return np.concatenate([counts, [16384]])
    counts = rng.multinomial(512, np.full(E, 1.0 / E))
    return np.concatenate([counts, [64]])


@pytest.mark.parametrize("name", list(FULL_COUNTS))
def test_tile_trace_full_size_schedules_cover_every_tile_once(name):
    if not os.path.exists(TRACE_LIB):
        pytest.skip("no tile-trace build")
    from split_weight_expert_amd import ExpertStore, _lib, api
    from split_weight_expert_amd.moe import DTYPES
    dt, seed = FULL_COUNTS[name]
    H, I = 7168, 2048
    counts = _full_counts(name, seed)
    G, rows = len(counts), int(counts.sum())
    print(f"{name}: {G} groups, {rows} rows", flush=True)
    rng = np.random.default_rng(seed)
    store = ExpertStore(H, I, DTYPES[dt], [1], device=DEV)
    store.load(0, 0, *[torch.from_numpy(rng.standard_normal(s).astype(np.float32) / np.sqrt(s[1])).to(DEV)
                       for s in ((I, H), (I, H), (H, I))])
    table = store.table([(0, 0)] * G, DEV)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(DEV)
    x = torch.randn(rows, H, device=DEV).to(torch.bfloat16)
    if dt == "fp8":
        xq = torch.empty(rows, H, dtype=torch.uint8, device=DEV)
        xs = torch.empty(rows, H // 128, dtype=torch.float32, device=DEV)
        api.quantize_tokens_fp8(x, xq, xs)
        x, x_scale, wcode = xq, xs, api.FP8_E4M3
    else:
        x_scale, wcode = None, api.BF16
    ws = torch.empty(api.workspace_bytes(api.OP_GROUPED_FFN, rows, 1, G, H, I, wcode, 0), dtype=torch.uint8,
                     device=DEV)
    y = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    saved = _lib._lib
    _lib._lib = None
    try:
        _lib.load(TRACE_LIB)
        traces = {}
        for stage in (1, 2):
            api.diag_tile_trace_clear()
            api.moe_grouped_ffn_stage(stage, table, G, offsets, x, x_scale, H, I, wcode, y, ws)
            torch.cuda.synchronize()
            tr = api.diag_tile_trace_read()
            traces[stage] = tr[tr["t_end"] > 0]
    finally:
        _lib._lib = saved
    for stage, n_tiles in ((1, I // 128), (2, H // 256)):
        _coverage(traces[stage], counts, n_tiles)
        assert ((traces[stage]["xcd"] >= 0) & (traces[stage]["xcd"] < 8)).all()
        # thousands of tiles reach every compute unit of the device, each named once by (XCD, HW_ID)
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        units = np.unique(traces[stage]["xcd"].astype(np.int64) * 256 + traces[stage]["hw_id"])
        assert len(units) == n_cu, f"stage {stage}: {len(units)} distinct compute units of {n_cu}"
    del store, table, x, ws, y
    torch.cuda.empty_cache()
