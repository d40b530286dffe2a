"""Benchmark of one DWDP rank's MoE block on MI355X.

Default workload: the DeepSeek-R1-shaped MoE layer at an 8K-token bf16 prefill
chunk (T=8192, H=7168, I=2048, 256 routed experts top-8 + 1 shared expert,
64 experts resident and 192 in a prefetch slot set).  A step is one pass of
the block -- route + top-k, permute, grouped SwiGLU FFN over the split
buffers, combine -- on one batch already resident in HBM.  The layer-ahead
prefetch runs on a side stream and is measured separately (copy alone, and
its slowdown of the block when both run at once).

Prints one JSON line.  --gpus N with N > 1 exits: the library runs one rank on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-block TFLOP/s & tokens/s at 8K tokens; % of MFMA peak (HBM GB/s decode)"
PEAK_BF16 = 2.5e15          # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5.0e15           # dense fp8
PEAK_FP32 = 157.3e12
PEAK_HBM = 8.0e12           # bytes/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill8k_bf16")
    ap.add_argument("--legs", default="decode64_bf16,prefill16k_fp8",
                    help="further workloads measured after the main one and reported under 'legs' (comma "
                         "separated; empty for none): the decode weight-streaming and fp8 prefetch-overlap figures")
    ap.add_argument("--leg-steps", type=int, default=10, help="timed steps of each extra leg")
    ap.add_argument("--overlap-engines", default="kernel,hipmemcpy",
                    help="copy engines whose overlap with the block is measured (the first is the default engine)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="FFN seconds the oracle's timed sample covers")
    ap.add_argument("--no-prefetch", action="store_true", help="skip the prefetch / overlap measurement")
    ap.add_argument("--no-merge", action="store_true", help="skip the merge-copy ablation")
    ap.add_argument("--pipeline-layers", type=int, default=0,
                    help="also run this many layers back to back with ping-pong prefetch slots")
    ap.add_argument("--slot-sets", type=int, default=2,
                    help="prefetch slot sets of the pipeline measurement (2 = the pages' double buffer)")
    ap.add_argument("--copy-workgroups", type=int, default=48)
    ap.add_argument("--copy-engine", default="kernel", choices=["kernel", "hipmemcpy", "sdma"],
                    help="engine of the pipeline and smi measurements")
    ap.add_argument("--chunk-mib", type=float, default=0, help="prefetch slice size in MiB (default: the workload's 4)")
    ap.add_argument("--burst-at", default="",
                    help="paced prefetch: comma-separated stage boundaries (0 block start, 1 after route, 2 after "
                         "permute, 3 after GEMM1, 4 after GEMM2) at which equal parts of the slice plan are released")
    ap.add_argument("--occupancy-probe", action="store_true",
                    help="time the block beside idle spinning workgroups (torch.cuda._sleep) that only occupy "
                         "compute units: 1, 4 and 16 of them for the block's length, and 1 for a quarter of it")
    ap.add_argument("--mechanism-probe", action="store_true",
                    help="time the block beside streams that isolate parts of the copy's cost: a read-only stream "
                         "(the operand-stream probe over the source regions, 48 workgroups), a write-only stream (a "
                         "fill of the pull's bytes), and the copy on compute units masked off from the block's")
    ap.add_argument("--copy-streams", type=int, default=1,
                    help="deal the prefetch's source regions round-robin over this many copy streams (the kernel "
                         "engine splits --copy-workgroups between them)")
    ap.add_argument("--smi", action="store_true",
                    help="also sample GPU clock and power (amd-smi) while the block runs alone, beside the "
                         "copy and beside a one-workgroup copy")
    ap.add_argument("--shape-study", action="store_true",
                    help="also time the expert GEMMs under other row distributions with the same rows "
                         "(balanced, dense, sparse/dense parts of the routed one) and hipBLASLt (torch) on "
                         "contiguous operands of the same shapes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run the slice-copy kernel on BYTES bytes (HBM counter calibration) and exit")
    ap.add_argument("--operand-probe", action="store_true",
                    help="only run the library's operand-stream probe (global_load_lds into an LDS ring, one "
                         "512-thread workgroup per compute unit) over L2 hits, last-level-cache hits and HBM, and "
                         "its LDS read probe, print one JSON line and exit")
    ap.add_argument("--tile-trace", action="store_true",
                    help="only trace the workload's two expert-GEMM launches tile by tile and print their "
                         "timeline statistics as one JSON line (needs a library built with "
                         "-DDWDP_TILE_TRACE=1, loaded through DWDP_LIBRARY)")
    return ap.parse_args()


def operand_probe(reps=4):
    """Rates of the operand path (dwdp_diag_operand_stream) for each source of bytes, best of `reps`."""
    import torch

    from split_weight_expert_amd import api
    MiB = 1 << 20
    grid_full = 256
    buf = torch.ones(16 << 30, dtype=torch.uint8, device="cuda")
    # (name, span, stride, iters, grid, in_flight, cpol)
    cases = [
        ("L2 hits: every workgroup reads the same 1 MiB", MiB, 0, 200, grid_full, 3, 0),
        ("last-level-cache hits: 256 regions of 1 MiB, each read 200 times", MiB, MiB, 200, grid_full, 3, 0),
        ("HBM: 256 streams of 64 MiB, 3 steps in flight", 64 * MiB, 64 * MiB, 1, grid_full, 3, 0),
        ("HBM: the same, non-temporal loads", 64 * MiB, 64 * MiB, 1, grid_full, 3, 2),
        ("HBM: 5 steps in flight", 64 * MiB, 64 * MiB, 1, grid_full, 5, 0),
        ("HBM: 2 steps in flight", 64 * MiB, 64 * MiB, 1, grid_full, 2, 0),
        ("HBM: 1 step in flight", 64 * MiB, 64 * MiB, 1, grid_full, 1, 0),
        ("HBM: 128 workgroups (half the compute units), 128 MiB each", 128 * MiB, 128 * MiB, 1, 128, 3, 0),
        ("L2 hits: 1 step in flight", MiB, 0, 200, grid_full, 1, 0),
    ]
    out = []
    for name, span, stride, iters, grid, infl, cpol in cases:
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            api.diag_operand_stream(buf, span, stride, iters, grid, infl, cpol)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        nbytes = span * iters * grid
        row = dict(case=name, workgroups=grid, in_flight_steps=infl, step_bytes=32768, cpol=cpol, bytes=nbytes,
                   ms=best, gbps_total=nbytes / best / 1e6, gbps_per_workgroup=nbytes / grid / best / 1e6)
        log(f"{name}: {row['gbps_total']:.0f} GB/s ({row['gbps_per_workgroup']:.1f} per workgroup)")
        out.append(row)
    lds = []
    for waves in (4, 8, 16):
        for grid in (256, 1):
            api.diag_lds_read(grid, waves, 2000)                     # warm-up
            bpc, ghz = api.diag_lds_read(grid, waves, 20000)
            lds.append(dict(waves_per_workgroup=waves, workgroups=grid, bytes_per_clock_per_cu=bpc, shader_ghz=ghz))
            log(f"LDS reads, {waves} waves x {grid} workgroups: {bpc:.0f} B per clock per CU at {ghz:.2f} GHz")
    print(json.dumps(dict(operand_probe=out, lds_read=lds, note="best of %d launches, HIP events; LDS rate from "
                          "the shader-clock counter" % reps)), flush=True)


def tile_trace(cfg, warm=3):
    """Per-tile timeline of the two expert-GEMM launches of one block (tile-trace build)."""
    import torch

    from split_weight_expert_amd import api
    from split_weight_expert_amd.workload import DeviceLayer
    if "tile-trace=1" not in api.version():
        print(f"bench.py --tile-trace: {api.version()!r} is not a tile-trace build (build one with "
              "DWDP_EXTRA_FLAGS=-DDWDP_TILE_TRACE=1 split_weight_expert_amd/build.py --out ..., then set "
              "DWDP_LIBRARY)", file=sys.stderr)
        sys.exit(2)
    layer = DeviceLayer(cfg, torch.device("cuda:0"), sources=False, slot_sets=2)
    block, table = layer.block(), layer.table(1)
    b = block.buffers(cfg.T)
    def blocks(n):
        for _ in range(n):
            block.route(layer.x, layer.w_router, layer.bias, b)
            block.permute(layer.x, b)
            block.ffn(table, b)
            block.combine(b)

    blocks(warm)
    torch.cuda.synchronize()
    counts = np.diff(b.offsets.cpu().numpy().astype(np.int64))
    res = dict(workload=cfg.name, tick_ns=10)
    n_cu = 256
    for stage in (1, 2):
        # the traced launch follows busy blocks with no host wait between them, so that it runs at the
        # clock the block holds; the clear sits between them on the stream
        blocks(warm)
        api.diag_tile_trace_clear()
        block.ffn_stage(stage, table, b)
        torch.cuda.synchronize()
        tr = api.diag_tile_trace_read()
        bid = np.nonzero(tr["t_end"] > 0)[0]
        tr = tr[bid]
        t0 = int(tr["t_start"].min())
        st = (tr["t_start"] - t0) / 100.0            # 100 MHz counter -> us
        en = (tr["t_end"] - t0) / 100.0
        dur = en - st
        span = float(en.max())
        ma = (tr["rows"] + 31) // 32
        full = ma == ma.max()
        edges = np.arange(0.0, span + 10.0, 10.0)
        running = np.array([int(((st <= t) & (en > t)).sum()) for t in edges])
        inner = (edges >= 100.0) & (edges <= span - 100.0)
        busy_tail = edges[running >= n_cu - 6]
        clusters = tr["order"] // 32
        spread = []
        for c in np.unique(clusters):
            m = clusters == c
            if m.sum() == 32:
                spread.append(float(st[m].max() - st[m].min()))
        q = lambda a: [round(float(np.percentile(a, x)), 1) for x in (10, 50, 90)] if len(a) else None
        # per compute unit (XCD and HW_ID): the gap from one tile's end to the start of the next tile that
        # unit takes (workgroup exit, dispatch of the next, its schedule lookup)
        unit = tr["xcd"].astype(np.int64) * 256 + tr["hw_id"]
        gaps, per_unit = [], []
        for u in np.unique(unit):
            m = np.nonzero(unit == u)[0]
            o = m[np.argsort(st[m])]
            per_unit.append(len(o))
            gaps.extend((st[o[1:]] - en[o[:-1]]).tolist())
        gaps = np.asarray(gaps)
        res[f"gemm{stage}"] = dict(
            tiles=int(len(tr)), span_us=round(span, 1),
            full_tile_us=round(float(dur[full].mean()), 1), full_tiles=int(full.sum()),
            one_block_tile_us=round(float(dur[ma == 1].mean()), 1) if (ma == 1).any() else None,
            tile_us_by_active_blocks={int(m): [int((ma == m).sum()), round(float(dur[ma == m].mean()), 1)]
                                      for m in np.unique(ma)},
            cu_busy_mean=round(float(dur.sum() / (n_cu * span)), 3),
            cu_busy_inside_100us=round(float(running[inner].mean() / n_cu), 3) if inner.any() else None,
            tail_below_250_tiles_us=round(span - float(busy_tail.max()), 1) if len(busy_tail) else None,
            xcd_end_us=[round(float(en[tr["xcd"] == x].max()), 1) if (tr["xcd"] == x).any() else None
                        for x in range(8)],
            xcd_is_workgroup_mod_8=round(float((tr["xcd"] == bid % 8).mean()), 4),
            cluster_start_spread_us_p10_50_90=q(spread),
            compute_units=int(len(per_unit)), tiles_per_unit_min_max=[int(min(per_unit)), int(max(per_unit))],
            inter_tile_gap_us_mean=round(float(gaps.mean()), 2) if len(gaps) else None,
            inter_tile_gap_us_p10_50_90=q(gaps),
            single_mtile_group_tiles=int((tr["group_m_tiles"] == 1).sum()),
            rows_of_groups_traced=int(counts[np.unique(tr["group"])].sum()))
        log(f"GEMM{stage}: {res[f'gemm{stage}']}")
    print(json.dumps(dict(tile_trace=res, version=api.version())), flush=True)


def calibrate_copy(nbytes, reps=3):
    """A plain copy of known size through the library's slice-copy kernel (one source, 4 MiB slices)."""
    import torch

    from split_weight_expert_amd import api
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.prefetch_chunks(dst.data_ptr(), [(src.data_ptr(), 0, nbytes)], 4 << 20, engine=api.COPY_KERNEL,
                            max_workgroups=256, copy_stream=torch.cuda.current_stream())
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    ok = bool(torch.equal(src[-4096:], dst[-4096:]))
    print(json.dumps(dict(calibrate_copy_bytes=nbytes, ms=float(np.median(t)),
                          gbps=nbytes / float(np.median(t)) / 1e6, ok=ok)), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(cfg, budget_s):
    """The oracle (as it stands) on a bounded sample of the workload, scaled to the whole layer.

    Sample: routing and permutation of all T tokens, then the expert FFN of every row routed to
    experts 0, 1, 2, ... (in order, skipping empty ones) until `budget_s` seconds of FFN work have
    been timed.  The FFN time is scaled by total rows / sampled rows (the FFN is over 99% of the
    layer's FLOPs).  Weight generation is not timed.
    """
    import threadpoolctl

    import synth
    from oracle import moe as omoe

    x = synth.tokens(cfg)
    wr = synth.router_weight(cfg)
    b = synth.router_bias(cfg)
    t0 = time.perf_counter()
    logits, idx, w = omoe.route(x, wr, b, cfg.k)
    offsets, src, inv, counts = omoe.permute(idx, cfg.E, cfg.shared)
    t_route = time.perf_counter() - t0
    t_ffn, rows, chosen = 0.0, 0, []
    for e in range(cfg.E):
        if t_ffn >= budget_s:
            break
        if counts[e] == 0:
            continue
        wts = synth.expert_weights(cfg, e)
        r0, r1 = offsets[e], offsets[e + 1]
        t0 = time.perf_counter()
        wg, wu, wd = omoe.prepare_weights(*wts, cfg.dtype)
        X = omoe.prepare_tokens(x[src[r0:r1]], cfg.dtype)
        omoe.expert_ffn(X, wg, wu, wd, cfg.dtype)
        t_ffn += time.perf_counter() - t0
        rows += int(r1 - r0)
        chosen.append(e)
    total_rows = cfg.T * (cfg.k + cfg.shared)
    est = t_route + t_ffn * total_rows / rows
    info = threadpoolctl.threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=cfg.T / est, unit="tokens/s", cores=int(threads), kind="oracle",
                tflops=6 * cfg.H * cfg.I * total_rows / est / 1e12, cpu_model=model, cores_available=int(cores),
                blas=[f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)" for i in blas],
                precision="fp64 (the oracle's own arithmetic, on bf16-valued inputs)",
                measured_s=dict(route_permute=t_route, ffn_sample=t_ffn),
                extrapolation=dict(sampled_rows=rows, total_rows=total_rows, factor=total_rows / rows),
                sample=(f"routing + permutation of all {cfg.T} tokens ({t_route:.2f} s, measured) and the "
                        f"{cfg.dtype}-policy fp64 expert FFN of the {rows} rows routed to the {len(chosen)} "
                        f"non-empty experts among 0..{chosen[-1]} ({t_ffn:.2f} s, measured); the FFN time is "
                        f"extrapolated by {total_rows}/{rows} rows to the whole layer (the FFN is over 99% of "
                        f"its FLOPs); weight generation not timed"))


def gemm_source_hash() -> str:
    import hashlib
    with open(os.path.join(ROOT, "split_weight_expert_amd", "csrc", "gemm.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per GEMM1 launch from the committed counter summary, if it was taken on this kernel source.

    The summary (profiles/gemm1_<workload>_hbm_traffic.md) holds FETCH_SIZE + WRITE_SIZE per dispatch,
    each scaled by what the counter reads for a copy of known size, and the sha256 of gemm.hip at the
    time; a different source gives None.
    """
    import re
    path = os.path.join(ROOT, "profiles", f"gemm1_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    v = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not v or h.group(1) != gemm_source_hash():
        return None
    return int(v.group(1))


def roofline(cfg, g1_ms, rows, touched, peak):
    """Roofline of the dominant kernel, GEMM1 + SwiGLU (gemm_frag_kernel, 2/3 of the FLOPs and weight bytes).

    Algorithmic work per launch: 4*H*I FLOPs per permuted row, and the W13 record part of every touched
    group read once (weights only; permuted activations are implementation traffic).  Decode batches
    (fewer rows than 8 per expert) are bounded by HBM, prefill by the MFMA peak of the weight dtype;
    both fractions are reported.
    """
    g1_s = g1_ms / 1e3
    flops = 4 * cfg.H * cfg.I * rows
    eb = {"fp8": 1, "bf16": 2, "f32": 4}[cfg.dtype]
    wbytes = touched * 2 * cfg.I * cfg.H * eb
    if cfg.dtype == "fp8":
        wbytes += touched * (2 * cfg.I // 128) * (cfg.H // 128) * 4
    hbm = dict(achieved=wbytes / g1_s / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s")
    mfma = dict(achieved=flops / g1_s / 1e12, peak=peak / 1e12, unit="TFLOP/s")
    decode = cfg.T * cfg.k < cfg.E * 8
    main_, other = (hbm, mfma) if decode else (mfma, hbm)
    roof = dict(bound="hbm" if decode else "mfma", **main_)
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic = measured_traffic(cfg.name)
    roof["traffic"] = traffic
    roof["kernel"] = "gemm_frag_kernel, GEMM1 + SwiGLU epilogue"
    roof["algorithmic"] = dict(flops=flops, weight_bytes=wbytes)
    roof["other_bound"] = dict(bound="mfma" if decode else "hbm", **other, frac=other["achieved"] / other["peak"])
    if traffic:
        roof["traffic_over_algorithmic_bytes"] = traffic / wbytes
    return roof


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs one rank on one GPU (asked for {args.gpus} GPUs); runs across "
              "several GPUs are not implemented", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.operand_probe:
        operand_probe()
        return
    cfg = synth.get_config(args.workload)
    if args.tile_trace:
        tile_trace(cfg)
        return
    res = run_workload(cfg, args, args.steps, args.warmup, main=True)
    legs = [w for w in args.legs.split(",") if w and w != cfg.name]
    if legs:
        res["legs"] = {}
        for name in legs:
            torch.cuda.empty_cache()
            leg = run_workload(synth.get_config(name), args, args.leg_steps, min(args.warmup, 3), main=False)
            res["legs"][name] = leg
        # the gates of the other workloads, flat
        for name, leg in res["legs"].items():
            if name.startswith("decode"):
                res["decode_hbm_frac"] = leg["roofline"]["frac"]
                res["decode_gemm1_gbps"] = leg["roofline"]["achieved"]
                res["decode_ffn_weight_gbps"] = leg["weight_gbps_ffn"]
            if leg.get("prefetch"):
                first = leg["prefetch"][0]
                key = name.split("_")[0]
                res[f"{key}_overlap_slowdown"] = first["slowdown"]
                res[f"{key}_overlap_hidden"] = first["hidden"]
                res[f"{key}_overlap_engine"] = first["engine"]
            if name.endswith("fp8"):
                res["fp8_gemm1_frac"] = leg["roofline"]["frac"]
                res["fp8_ffn_frac"] = leg["frac_peak_ffn"]

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def run_workload(cfg, args, steps, warmup, main):
    """Build one synthetic layer on the GPU, time `steps` blocks, and measure the prefetch beside it (and,
    for the main workload, the optional studies).  The layer is freed before returning."""
    import torch

    from split_weight_expert_amd.workload import DeviceLayer

    dev = torch.device("cuda:0")
    want_prefetch = not args.no_prefetch and cfg.n_prefetch > 0
    log(f"setting up {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} dtype={cfg.dtype}")
    t0 = time.perf_counter()
    layer = DeviceLayer(cfg, dev, sources=want_prefetch,
                        slot_sets=max(2, args.slot_sets) if main and args.pipeline_layers > 0 else 2)
    log(f"layer resident in {time.perf_counter() - t0:.1f} s")
    block = layer.block()
    table = layer.table(1)
    x, wr, bias = layer.x, layer.w_router, layer.bias
    st = torch.cuda.current_stream()
    b = block.buffers(cfg.T)

    def step(ev=None):
        if ev is not None:
            ev[0].record(st)
        block.route(x, wr, bias, b)
        if ev is not None:
            ev[1].record(st)
        block.permute(x, b)
        if ev is not None:
            ev[2].record(st)
        block.ffn_stage(1, table, b)
        if ev is not None:
            ev[3].record(st)
        block.ffn_stage(2, table, b)
        if ev is not None:
            ev[4].record(st)
        block.combine(b)
        if ev is not None:
            ev[5].record(st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / steps * 1e3
    # Stage times: the same steps again with an event at every stage boundary.  Those events (six per
    # step) cost about 0.5% of a step, so they stay out of the timed loop above.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ["route", "permute", "gemm1_swiglu", "gemm2", "combine"]
    stage_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    step_ev_ms = [e[0].elapsed_time(e[5]) for e in evs]      # each step between its first and last event
    log(f"{cfg.name}: step {ms_step:.3f} ms; stages " + ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))

    counts = np.diff(b.offsets.cpu().numpy())
    rows = int(counts.sum())
    routed = np.sort(counts[:cfg.E].astype(np.float64))
    # Gini coefficient of the routed experts' row counts (0: every expert the same load)
    gini = float((2 * np.arange(1, cfg.E + 1) - cfg.E - 1) @ routed / (cfg.E * routed.sum())) if routed.sum() else 0.0
    load = dict(max_rows=int(routed[-1]), median_rows=float(np.median(routed)), min_rows=int(routed[0]),
                empty_experts=int((routed == 0).sum()), gini=gini)
    touched = int((counts[:cfg.E] > 0).sum()) + cfg.shared
    flops_ffn = 6 * cfg.H * cfg.I * rows
    flops_total = flops_ffn + 2 * cfg.T * cfg.H * cfg.E
    peak = {"bf16": PEAK_BF16, "fp8": PEAK_FP8, "f32": PEAK_FP32}[cfg.dtype]
    wbytes = layer.store.rec
    ffn_s = (stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]) / 1e3
    res_roof = roofline(cfg, stage_ms["gemm1_swiglu"], rows, touched, peak)
    head = dict(metric=METRIC, value=cfg.T / (ms_step / 1e3), unit="tokens/s", n_gpus=1, steps=steps,
                warmup=warmup, ms_per_step=ms_step, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype=cfg.dtype, data="synthetic (seeded; no trained weights)",
                config=dict(workload=f"{cfg.name}: {cfg.note}", T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k,
                            shared=cfg.shared, local_experts=cfg.n_local, prefetch_experts=cfg.n_prefetch,
                            parallelism="one rank of DWDP (single GPU)"))
    res = head if main else dict(value=head["value"], unit="tokens/s", ms_per_step=ms_step, steps=steps,
                                 dtype=cfg.dtype, config=head["config"])
    res.update(tflops_block=flops_total / (ms_step / 1e3) / 1e12, tflops_ffn=flops_ffn / ffn_s / 1e12,
               frac_peak_ffn=flops_ffn / ffn_s / peak, weight_gbps_ffn=touched * wbytes / ffn_s / 1e9,
               frac_hbm_ffn=touched * wbytes / ffn_s / PEAK_HBM,
               experts_touched=touched, rows=rows, expert_load=load, stage_ms=stage_ms,
               step_ms_events=dict(p10=float(np.percentile(step_ev_ms, 10)), median=float(np.median(step_ev_ms)),
                                   p90=float(np.percentile(step_ev_ms, 90))),
               roofline=res_roof)

    if want_prefetch:
        engines = [e for e in args.overlap_engines.split(",") if e]
        res["prefetch"] = [measure_prefetch(layer, block, step, args, cfg, ms_step, eng) for eng in engines]
        if main and args.smi:
            res["prefetch"][0]["smi"] = measure_smi(layer, step, args, cfg)
    if main and args.pipeline_layers > 0 and want_prefetch:
        res["pipeline"] = measure_pipeline(layer, block, step, args, cfg, res["prefetch"][0])
    if main and not args.no_merge and cfg.n_prefetch > 0:
        res["merge_ablation"] = measure_merge(layer, block, cfg, b, stage_ms)
    if main and args.shape_study:
        res["shape_study"] = measure_shapes(layer, block, cfg, b)
    if main and args.occupancy_probe:
        res["occupancy_probe"] = measure_occupancy(step, cfg)
    if main and args.mechanism_probe and want_prefetch:
        res["mechanism_probe"] = measure_mechanisms(layer, block, table, b, cfg)
    del layer, block, b, table
    torch.cuda.synchronize()
    return res


def _median_ms(fn, reps=5, warm=2):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def measure_shapes(layer, block, cfg, b):
    """Where the expert GEMMs' time goes, from the row distribution alone.

    The same grouped FFN entry point runs on offsets other than the routed ones (every call keeps
    rows == offsets[G], using the first rows of perm_src):
      * routed:   the layer's own routing;
      * balanced: every routed expert R/E rows, the shared expert T;
      * dense:    k routed experts with T rows each plus the shared expert, so the rows are the
                  routed ones' but the weights touched are few and reused from cache;
      * split:    the routed counts cut at a row threshold into the sparse groups alone and the
                  others alone (their times add up to the routed time when the two kinds do not
                  overlap).
    Reference (bf16 only): hipBLASLt through torch on contiguous operands of the balanced shapes --
    a batched product over the E experts of R/E rows plus one product for the shared expert, for
    GEMM1 ([rows, H] x [H, 2I]) and GEMM2 ([rows, I] x [I, H]); no pointer table, no SwiGLU.
    """
    import torch

    from split_weight_expert_amd import api

    G = cfg.E + cfg.shared
    table = layer.table(1)
    routed = np.diff(b.offsets.cpu().numpy()).astype(np.int64)
    saved = b.offsets.clone()
    fl1 = 4 * cfg.H * cfg.I

    def run(counts):
        counts = np.asarray(counts, dtype=np.int64)
        offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(layer.device)
        rows = int(counts.sum())
        ps = b.perm_src[:rows]

        def stage(s):
            api.moe_grouped_ffn_tokens(s, table, G, offs, ps, b.x_tokens, b.x_q_scale, cfg.H, cfg.I, block.w_dtype,
                                       b.y_perm, b.ws_ffn)
        stage(1)
        g1 = _median_ms(lambda: stage(1))
        g2 = _median_ms(lambda: stage(2))   # reads the A that the last GEMM1 left in the workspace
        return dict(rows=rows, groups=int((counts > 0).sum()), gemm1_ms=g1, gemm2_ms=g2,
                    gemm1_tflops=fl1 * rows / g1 / 1e9, gemm2_tflops=fl1 / 2 * rows / g2 / 1e9)

    out = {"routed": run(routed)}
    if cfg.R % cfg.E == 0:
        bal = np.full(G, cfg.R // cfg.E, dtype=np.int64)
        bal[cfg.E:] = cfg.T
        out["balanced"] = run(bal)
    dense = np.zeros(G, dtype=np.int64)
    dense[:cfg.k] = cfg.T
    dense[cfg.E:] = cfg.T
    out["dense"] = run(dense)
    splits = []
    for thr in (32, 64):
        sp = np.where(routed <= thr, routed, 0)
        sp[cfg.E:] = 0
        if sp.sum() == 0:
            continue
        a, d = run(sp), run(routed - sp)
        splits.append(dict(max_rows=thr, sparse=a, rest=d, sum_gemm1_ms=a["gemm1_ms"] + d["gemm1_ms"],
                           sum_gemm2_ms=a["gemm2_ms"] + d["gemm2_ms"]))
    out["split"] = splits
    b.offsets.copy_(saved)

    if cfg.dtype == "bf16" and cfg.R % cfg.E == 0:
        n = cfg.R // cfg.E
        dev, bf = layer.device, torch.bfloat16
        ref = {}
        for name, K, N in (("gemm1", cfg.H, 2 * cfg.I), ("gemm2", cfg.I, cfg.H)):
            a = torch.randn(cfg.E, n, K, device=dev, dtype=bf)
            w = (torch.randn(cfg.E, K, N, device=dev) / math.sqrt(K)).to(bf)   # contiguous [E, K, N]
            o = torch.empty(cfg.E, n, N, device=dev, dtype=bf)
            xs = torch.randn(cfg.T, K, device=dev, dtype=bf)
            ws = (torch.randn(K, N, device=dev) / math.sqrt(K)).to(bf)
            os_ = torch.empty(cfg.T, N, device=dev, dtype=bf)

            def f():
                torch.bmm(a, w, out=o)
                torch.matmul(xs, ws, out=os_)
            ms = _median_ms(f)
            ms_dense = _median_ms(lambda: torch.matmul(xs, ws, out=os_))
            rows = cfg.E * n + cfg.T
            ref[name] = dict(ms=ms, tflops=2 * K * N * rows / ms / 1e9, dense_T_ms=ms_dense,
                             dense_T_tflops=2 * K * N * cfg.T / ms_dense / 1e9)
            del a, w, o, xs, ws, os_
        torch.cuda.empty_cache()
        out["hipblaslt_balanced"] = ref
    return out


def measure_merge(layer, block, cfg, b, stage_ms):
    """The baseline the pointer table replaces: merge every group's record into one contiguous buffer
    with a device-to-device copy (the library's slice-copy kernel on the whole GPU), then run the same
    grouped FFN on it.  Reports the merge time next to the FFN on the split buffers."""
    import torch

    from split_weight_expert_amd import api

    store = layer.store
    G = cfg.E + cfg.shared
    rec = store.rec
    merged = torch.empty(G * rec, dtype=torch.uint8, device=layer.device)
    # group order: resident experts, prefetched experts, then the shared expert (resident slot n_local)
    srcs = [(store.buffers[0].data_ptr(), 0, cfg.n_local * rec),
            (store.buffers[1].data_ptr(), cfg.n_local * rec, cfg.n_prefetch * rec)]
    if cfg.shared:
        srcs.append((store.buffers[0].data_ptr() + cfg.n_local * rec, cfg.E * rec, rec))
    st = torch.cuda.current_stream()
    table_m = api.table_to_device(api.fill_expert_table([merged.data_ptr()], [0] * G, list(range(G)), cfg.H, cfg.I,
                                                        store.w_dtype), layer.device)

    def merge():
        api.prefetch_chunks(merged.data_ptr(), srcs, cfg.chunk_bytes, engine=api.COPY_KERNEL, max_workgroups=256,
                            copy_stream=st)

    merge()
    block.ffn_stage(1, table_m, b)
    block.ffn_stage(2, table_m, b)
    torch.cuda.synchronize()
    y_merged = b.y_perm.clone()
    t_merge, t_ffn = [], []
    for _ in range(5):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(st)
        merge()
        e[1].record(st)
        block.ffn_stage(1, table_m, b)
        block.ffn_stage(2, table_m, b)
        e[2].record(st)
        torch.cuda.synchronize()
        t_merge.append(e[0].elapsed_time(e[1]))
        t_ffn.append(e[1].elapsed_time(e[2]))
    # the FFN alone on the merged buffer (no merge right before it)
    t_alone = []
    for _ in range(5):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(st)
        block.ffn_stage(1, table_m, b)
        block.ffn_stage(2, table_m, b)
        e[1].record(st)
        torch.cuda.synchronize()
        t_alone.append(e[0].elapsed_time(e[1]))
    # the same FFN through the split buffers must give the same bits
    block.ffn_stage(1, layer.table(1), b)
    block.ffn_stage(2, layer.table(1), b)
    torch.cuda.synchronize()
    same = bool(torch.equal(y_merged, b.y_perm))
    ffn_split = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]
    m, f = float(np.median(t_merge)), float(np.median(t_ffn))
    del merged
    return dict(merged_bytes=G * rec, merge_ms=m, merge_gbps=G * rec / m / 1e6, ffn_ms_after_merge=f,
                ffn_ms_merged=float(np.median(t_alone)), ffn_ms_split=ffn_split,
                merge_plus_ffn_over_split=(m + f) / ffn_split, same_result=same,
                note="merge = one slice-copy launch over all groups' records (256 workgroups)")


def measure_pipeline(layer, block, step, args, cfg, pf):
    """L layers back to back through the library's DWDPPipeline (DWDP paper summary §2): layer l reads
    prefetch slot set l % 2 while the copy stream fills slot set (l + 1) % 2 with the next layer's
    non-local experts; a pull waits for the last layer that read its slot set and a layer waits for the
    pull that filled its own.  Every layer here has the same weights and reads the same input (the
    source regions stand in for the peers of every layer, so each pull moves the same bytes), and only
    the MoE block computes (no attention): the copy has the block alone to hide behind, the
    conservative case.
    """
    import torch

    from split_weight_expert_amd import DWDPPipeline, LayerWeights, api

    L = args.pipeline_layers
    engine = {"kernel": api.COPY_KERNEL, "hipmemcpy": api.COPY_HIPMEMCPY, "sdma": api.COPY_SDMA}[args.copy_engine]
    chunk = int(args.chunk_mib * (1 << 20)) if args.chunk_mib else cfg.chunk_bytes
    comp = torch.cuda.current_stream()
    N = max(2, args.slot_sets)
    pipe = DWDPPipeline(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, cfg.n_local, layer.device,
                        slot_sets=layer.store.buffers[1:1 + N], chunk_bytes=chunk, engine=engine,
                        max_workgroups=args.copy_workgroups)
    pipe.block = block
    lw = LayerWeights(layer.w_router, layer.bias, layer.store.buffers[0], layer.sources)
    outs = [torch.empty(cfg.T, cfg.H, dtype=layer.x.dtype, device=layer.device) for _ in range(2)]

    def run():
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # timed from the start of layer 0's block (after the first pull, which nothing could hide)
        pipe.forward(layer.x, [lw] * L, outputs=[outs[l % 2] for l in range(L)], chain=False,
                     before_compute=lambda l: start.record(comp) if l == 0 else None)
        end.record(comp)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    run()
    t = float(np.median([run() for _ in range(3)]))
    # compute alone per layer
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(L):
        step()
    e1.record()
    torch.cuda.synchronize()
    tc = e0.elapsed_time(e1) / L
    tp = pf["copy_ms"]
    # both slot sets now hold the sources' bytes: spot-check one record of each
    per = cfg.n_prefetch // cfg.n_sources
    ok = all(bool(torch.equal(layer.store.record(k, per + 1), layer.src_store.record(1, 1))) for k in range(1, N + 1))
    model = max(tc, tp / (N - 1))
    return dict(layers=L, slot_sets=N, engine=args.copy_engine, chunk_bytes=chunk, ms_per_layer=t / L,
                compute_ms_per_layer=tc, copy_ms_alone=tp, max_tc_tp=max(tc, tp), model_ms=model,
                layer_over_model=(t / L) / model, layer_over_compute=(t / L) / tc, record_check=ok,
                note="DWDPPipeline over the MoE block only (no attention); with N slot sets the pull of layer "
                     "l+N-1 overlaps layers l..l+N-2; model = max(compute, copy / (N-1)); timed from layer 0's "
                     "block to the end of the last layer")


def burst_parts(sources, chunk, n):
    """The slice plan's rounds cut into n equal parts: part j is the list of (src, dst_offset, bytes) that,
    planned on its own, gives the rounds [R*j/n, R*(j+1)/n) of the whole plan (R rounds), in the same
    order, so the parts together copy the same slices in the same order."""
    rounds = max(-(-s[2] // chunk) for s in sources)
    parts = []
    for j in range(n):
        r0, r1 = rounds * j // n, rounds * (j + 1) // n
        part = []
        for src, off, nbytes in sources:
            a, e = min(nbytes, r0 * chunk), min(nbytes, r1 * chunk)
            if e > a:
                part.append((src + a, off + a, e - a))
        parts.append(part)
    return parts


def measure_prefetch(layer, block, step, args, cfg, ms_block, engine_name):
    """Copy of the next layer's non-local experts into slot set 2: alone, and beside the block.

    The block's time with and without the copy comes from the same protocol: from an idle GPU, an event
    `start` on the compute stream, one block, an event `b_end`; with the copy, the copy stream waits on
    `start` and the copy is enqueued right after the block.  The slowdown is the ratio of the two
    medians over the same number of repetitions."""
    import torch

    from split_weight_expert_amd import api

    engine = {"kernel": api.COPY_KERNEL, "hipmemcpy": api.COPY_HIPMEMCPY, "sdma": api.COPY_SDMA}[engine_name]
    dst = layer.store.buffers[2].data_ptr()
    nbytes = sum(s[2] for s in layer.sources)
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    n_cs = max(1, min(args.copy_streams, len(layer.sources)))
    extra = [torch.cuda.Stream() for _ in range(n_cs - 1)]

    chunk = int(args.chunk_mib * (1 << 20)) if args.chunk_mib else cfg.chunk_bytes

    # Paced release (--burst-at): part j of the plan is released when the block passes stage boundary
    # bursts[j] (an event on the compute stream).
    bursts = [int(v) for v in args.burst_at.split(",") if v != ""]
    assert all(0 <= v <= 4 for v in bursts), "--burst-at takes stage boundaries 0..4"
    parts = burst_parts(layer.sources, chunk, len(bursts)) if bursts else []

    def copy(wait=None, done=None, sources=None):
        # stream i copies source regions i, i + n, ...; the other streams join cs before `done`
        sources = layer.sources if sources is None else sources
        for st in extra:
            st.wait_stream(cs)
        for i, st in enumerate([cs] + extra):
            api.prefetch_chunks(dst, sources[i::n_cs], chunk, engine=engine,
                                max_workgroups=max(1, args.copy_workgroups // n_cs), copy_stream=st, wait_event=wait,
                                done_event=done if n_cs == 1 else None)
        if n_cs > 1:
            for st in extra:
                cs.wait_stream(st)
            if done is not None:
                done.record(cs)

    reps = max(5, min(args.steps, 10))
    # copy alone
    copy()
    torch.cuda.synchronize()
    # host time to enqueue the whole plan (one launch for the kernel engine, one call per slice otherwise)
    h0 = time.perf_counter()
    copy()
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_copy = []
    for _ in range(reps):
        e0.record(cs)
        copy()
        e1.record(cs)
        torch.cuda.synchronize()
        t_copy.append(e0.elapsed_time(e1))

    def single(with_copy):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        c_end = torch.cuda.Event(enable_timing=True)
        step(ev)
        start, b_end = ev[0], ev[5]
        # the block is enqueued first: the SDMA engine's host enqueue blocks for a while and must not
        # delay the block's launch
        if with_copy and bursts:
            for j, (at, part) in enumerate(zip(bursts, parts)):
                copy(wait=ev[at], done=c_end if j == len(parts) - 1 else None, sources=part)
        elif with_copy:
            copy(wait=start, done=c_end)
        torch.cuda.synchronize()
        tb = start.elapsed_time(b_end)
        return tb, (start.elapsed_time(c_end) if with_copy else None)

    # the block alone first (each from an idle GPU, as in the copy's leg, but not right after a copy: a
    # copy that runs on alone leaves the block's operands evicted from the caches), then beside the copy
    t_alone = [single(False)[0] for _ in range(reps)]
    t_blk, t_cp = [], []
    for _ in range(reps):
        tb, tc = single(True)
        t_blk.append(tb)
        t_cp.append(tc)
    # the destination now holds layer l+1's experts: spot-check one record byte-for-byte
    per = cfg.n_prefetch // cfg.n_sources
    ok = bool(torch.equal(layer.store.record(2, per + 1), layer.src_store.record(1, 1)))
    c_alone = float(np.median(t_copy))
    alone, beside, cbeside = float(np.median(t_alone)), float(np.median(t_blk)), float(np.median(t_cp))
    n_chunks = len(api.prefetch_plan(layer.sources, chunk))
    log(f"{cfg.name}: prefetch ({engine_name}{', bursts at ' + args.burst_at if bursts else ''}) copy "
        f"{c_alone:.2f} ms alone; block {alone:.3f} -> {beside:.3f} ms beside it ({beside / alone - 1:+.1%}), "
        f"copy done at {cbeside:.2f} ms")
    return dict(engine=engine_name, workgroups=args.copy_workgroups if engine_name == "kernel" else None,
                bursts_at=bursts or None,
                streams=n_cs, bytes=nbytes, chunk_bytes=chunk, n_chunks=n_chunks,
                host_enqueue_us_per_chunk=host_s * 1e6 / max(1, n_chunks),
                copy_ms=c_alone, copy_gbps=nbytes / c_alone / 1e6,
                block_ms_alone=alone, block_ms_with_copy=beside, block_ms_loop=ms_block,
                copy_ms_with_block=cbeside, layer_ms_overlapped=float(np.median([max(a, b) for a, b in
                                                                                 zip(t_blk, t_cp)])),
                slowdown=beside / alone - 1.0, hidden=bool(cbeside <= beside), reps=reps, record_check=ok,
                note="stand-in source regions sit in the same HBM, so the copy reads and writes locally")


def measure_occupancy(step, cfg, reps=8):
    """The block beside workgroups that do nothing but occupy compute units.

    torch.cuda._sleep launches one single-thread workgroup that spins for a number of GPU clock cycles and
    touches no memory.  n of them go on n side streams, started with the block (the streams wait on the
    block's first event); the block is timed with the single-step protocol of the prefetch leg.  Their
    cost is what any concurrent kernel costs the block by its presence on the compute units alone."""
    import torch

    comp = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in range(16)]

    def single(n, cycles):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(comp)
        for st in streams[:n]:
            st.wait_event(ev[0])
            with torch.cuda.stream(st):
                torch.cuda._sleep(cycles)
        step(ev)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[5])

    alone = float(np.median([single(0, 0) for _ in range(reps)]))
    # calibrate the spin: cycles per millisecond of the clock _sleep counts
    probe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe[0].record(comp)
    torch.cuda._sleep(10_000_000)
    probe[1].record(comp)
    torch.cuda.synchronize()
    per_ms = 10_000_000 / max(probe[0].elapsed_time(probe[1]), 1e-3)
    out = dict(block_ms_alone=alone, sleep_cycles_per_ms=per_ms, cases=[])
    for n, frac in ((1, 1.2), (4, 1.2), (16, 1.2), (1, 0.25)):
        ms = alone * frac
        t = float(np.median([single(n, int(ms * per_ms)) for _ in range(reps)]))
        out["cases"].append(dict(workgroups=n, spin_ms=ms, block_ms=t, slowdown=t / alone - 1.0))
        log(f"{cfg.name}: block beside {n} idle workgroup(s) spinning {ms:.1f} ms: {alone:.3f} -> {t:.3f} ms "
            f"({t / alone - 1:+.1%})")
    return out


def _hip_runtime():
    """The HIP runtime this process already uses (torch's), for calls that torch does not expose."""
    import ctypes
    path = [line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line][0]
    return ctypes.CDLL(path)


def cu_masked_stream(hip, mask_words):
    """A stream whose kernels run only on the compute units set in mask_words (hipExtStreamCreateWithCUMask;
    default priority)."""
    import ctypes

    import torch
    arr = (ctypes.c_uint32 * len(mask_words))(*mask_words)
    s = ctypes.c_void_p()
    fn = hip.hipExtStreamCreateWithCUMask
    fn.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
    rc = fn(ctypes.byref(s), len(mask_words), arr)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask returned {rc}")
    return torch.cuda.ExternalStream(s.value)


def measure_mechanisms(layer, block, table, b, cfg, reps=8, copy_bits=8):
    """The block (single-step protocol: an event, the block, an event, from an idle GPU; medians) beside
    streams that each keep one property of the prefetch copy:
      read_only   the operand-stream probe reading the three source regions, 16 workgroups each on three
                  streams (48, the copy kernel's default), with non-temporal loads like the copy's and with
                  loads that allocate in L2: its reads, no writes;
      write_only  a fill of the pull's bytes in the other slot set: its writes, no reads;
      cu_split    the copy kernel itself (3 workgroups per compute unit it may use) on a stream masked to
                  copy_bits of every 32 compute units, and the block on a stream masked to the others, so
                  that no compute unit holds both."""
    import torch

    from split_weight_expert_amd import api
    x, wr, bias = layer.x, layer.w_router, layer.bias
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    dst = layer.store.buffers[2]
    pull = sum(n for _, _, n in layer.sources)

    def block_on(s):
        block.route(x, wr, bias, b, s)
        block.permute(x, b, s)
        block.ffn_stage(1, table, b, s)
        block.ffn_stage(2, table, b, s)
        block.combine(b, s)

    def single(s, extra=None, side_streams=()):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        if extra is not None:
            for ss in side_streams:
                ss.wait_event(e0)
            extra(side_streams)
        block_on(s)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def timed(fn, streams):
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(streams[0])
        for ss in streams[1:]:
            ss.wait_event(e0)
        fn(streams)
        ends = []
        for ss in streams:
            e = torch.cuda.Event(enable_timing=True)
            e.record(ss)
            ends.append(e)
        torch.cuda.synchronize()
        return max(e0.elapsed_time(e) for e in ends)

    med = lambda f: float(np.median([f() for _ in range(reps)]))
    src_views = []
    for ptr, _, n in layer.sources:
        span = (n // 16) // 32768 * 32768
        src_views.append((ptr, span))
    src_tensors = {}
    for buf in layer.src_store.buffers:
        src_tensors[buf.data_ptr()] = buf

    sides = [torch.cuda.Stream() for _ in src_views]

    def read_only(cpol):
        def go(streams):
            for (ptr, span), ss in zip(src_views, streams):
                api.diag_operand_stream(src_tensors[ptr], span, span, 1, 16, 3, cpol, ss)
        return go

    def write_only(streams):
        with torch.cuda.stream(streams[0]):
            dst[:pull].zero_()

    out = dict(workload=cfg.name, reps=reps)
    single(comp)
    alone = med(lambda: single(comp))
    out["block_ms_alone"] = alone
    read_bytes = sum(sp * 16 for _, sp in src_views)
    for name, fn, nbytes, ss in (("read_only_nontemporal", read_only(2), read_bytes, sides),
                                 ("read_only_l2_allocating", read_only(0), read_bytes, sides),
                                 ("write_only", write_only, pull, [side])):
        fn(ss)
        torch.cuda.synchronize()
        t_side = med(lambda: timed(fn, ss))
        t = med(lambda: single(comp, fn, ss))
        out[name] = dict(bytes=nbytes, side_ms_alone=t_side, side_gbps=nbytes / t_side / 1e6, block_ms=t,
                         slowdown=t / alone - 1.0)
        log(f"{cfg.name}: block beside a {name.replace('_', '-')} stream ({nbytes / 1e9:.2f} GB, {t_side:.2f} ms alone): "
            f"{alone:.3f} -> {t:.3f} ms ({t / alone - 1:+.1%})")
    # compute units split between the block and the copy
    hip = _hip_runtime()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    words = (ncu + 31) // 32
    cmask = (1 << copy_bits) - 1
    comp_m = cu_masked_stream(hip, [0xFFFFFFFF & ~cmask] * words)
    copy_m = cu_masked_stream(hip, [cmask] * words)
    n_copy_cu = copy_bits * words

    def copy(streams):
        api.prefetch_chunks(dst.data_ptr(), layer.sources, cfg.chunk_bytes, engine=api.COPY_KERNEL,
                            max_workgroups=3 * n_copy_cu, copy_stream=streams[0])

    single(comp_m)
    masked_alone = med(lambda: single(comp_m))
    copy([copy_m])
    torch.cuda.synchronize()
    copy_alone = med(lambda: timed(copy, [copy_m]))
    beside = med(lambda: single(comp_m, copy, [copy_m]))
    out["cu_split"] = dict(copy_cus=n_copy_cu, block_cus=ncu - n_copy_cu, copy_workgroups=3 * n_copy_cu,
                           block_ms_alone_masked=masked_alone, copy_ms_alone_masked=copy_alone,
                           block_ms_beside=beside, slowdown_vs_masked=beside / masked_alone - 1.0,
                           slowdown_vs_all_cus=beside / alone - 1.0)
    log(f"{cfg.name}: block on {ncu - n_copy_cu} CUs {masked_alone:.3f} ms alone ({masked_alone / alone - 1:+.1%} vs all "
        f"CUs), {beside:.3f} ms beside the copy on the other {n_copy_cu} ({beside / masked_alone - 1:+.1%}); copy alone "
        f"there {copy_alone:.2f} ms")
    return out


def measure_smi(layer, step, args, cfg, secs=2.5):
    """GPU clock and socket power (amd-smi, sampled from a thread) while the block runs back to back:
    alone, beside the prefetch copy (args.copy_workgroups) started with every block, and beside one
    long copy of a single workgroup.  Tells a clock (DVFS) slowdown from a contention one."""
    import subprocess
    import threading

    import torch

    from split_weight_expert_amd import api

    dst = layer.store.buffers[2].data_ptr()
    cs = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            t0 = time.time()
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                g = json.loads(r.stdout)["gpu_data"][0]
                clk = [g["clock"][k]["clk"]["value"] for k in g["clock"] if k.startswith("gfx_")]
                samples.append(((t0 + time.time()) / 2, float(g["power"]["socket_power"]["value"]),
                                float(np.mean(clk))))
            except Exception:
                return

    def copy(wg):
        s = torch.cuda.Event()
        s.record(comp)
        api.prefetch_chunks(dst, layer.sources, cfg.chunk_bytes, engine=api.COPY_KERNEL, max_workgroups=wg,
                            copy_stream=cs, wait_event=s)

    def phase(name, with_copy):
        t0 = time.time()
        ms = []
        while time.time() - t0 < secs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if with_copy > 1:
                copy(with_copy)
            elif with_copy == 1 and cs.query():
                copy(1)                               # one workgroup, kept running beside the blocks
            e0.record(comp)
            step()
            e1.record(comp)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
            if with_copy > 1:
                cs.synchronize()
        torch.cuda.synchronize()
        t1 = time.time()
        sel = [x for x in samples if t0 + 0.3 < x[0] < t1]
        return name, dict(block_ms=float(np.median(ms)), blocks=len(ms), samples=len(sel),
                          power_w=float(np.median([x[1] for x in sel])) if sel else None,
                          gfx_mhz=float(np.median([x[2] for x in sel])) if sel else None)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(1.0)
    out = dict([phase("alone", 0), phase("beside_copy", args.copy_workgroups), phase("beside_1wg_copy", 1)])
    stop.set()
    th.join(timeout=15)
    log("smi: " + ", ".join(f"{k} {v['block_ms']:.3f} ms {v['gfx_mhz']} MHz {v['power_w']} W" for k, v in out.items()))
    return out


if __name__ == "__main__":
    main()
