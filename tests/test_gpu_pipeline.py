"""The layer-ahead prefetch pipeline (DWDPPipeline) against the per-layer oracle, with delays injected.

L = 4 distinct seeded layers, each with its own resident records and its own stand-in source
allocations for its non-local experts, run back to back: layer l reads prefetch slot set l % N while
the copy stream fills the other sets with the next layers' experts (N = 2, the pages' double buffer,
DWDP paper summary §2; §4.3.2 slices; and N = 3).
Delays are injected at enqueue time with torch.cuda._sleep on the copy stream (each pull starts late,
so a layer that did not wait for its copy would read the weights of layer l-2 left in its slot set)
and on the compute stream (each layer runs late, so a pull that did not wait for the last reader would
overwrite the weights under it).  Every layer's routing must be the oracle's top-k of the GPU's own
logits (bit-exact) and its output must match the oracle's layer applied to the GPU's input of that
layer, within the dtype's tolerance.  A second forward call reuses the slot sets (the first pull must
wait for the previous call's last reader).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as omoe
from synth.configs import shrink
from tests.gpu_util import assert_close, need_gpu, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
L = 4
SLEEP = 20_000_000          # cycles of torch.cuda._sleep (a few ms)

CASES = {
    "f32": ("tiny_f32", dict(T=96, H=256, I=128, E=8, k=2, shared=1, n_local=3, n_sources=1)),
    "bf16": ("prefill8k_bf16", dict(T=160, H=512, I=256, E=12, k=3, shared=1, n_local=4, n_sources=2)),
}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def build_layers(cfg):
    """Per layer: host weights (for the oracle) and LayerWeights on the device."""
    from split_weight_expert_amd import ExpertStore, LayerWeights
    from split_weight_expert_amd.moe import DTYPES, act_dtype
    wd = DTYPES[cfg.dtype]
    adt = act_dtype(wd)
    n_pre = cfg.E - cfg.n_local
    per = -(-n_pre // cfg.n_sources)
    host, dev, stores = [], [], []
    for l in range(L):
        experts = [synth.expert_weights(cfg, e, layer=l) for e in range(cfg.E)]
        shared = synth.expert_weights(cfg, cfg.E, layer=l) if cfg.shared else None
        wr = synth.router_weight(cfg, l)
        b = synth.router_bias(cfg, l)
        # resident buffer, then one buffer per stand-in source region
        sizes = [cfg.n_local + cfg.shared] + [min(per, n_pre - i * per) for i in range(cfg.n_sources)]
        st = ExpertStore(cfg.H, cfg.I, wd, sizes, device=DEV)

        def put(buf, slot, ws):
            ts = [torch.from_numpy(a).to(DEV) for a in ws]
            if cfg.dtype != "fp8":
                ts = [t.to(adt) for t in ts]
            st.load(buf, slot, *ts)
        for e in range(cfg.n_local):
            put(0, e, experts[e])
        if cfg.shared:
            put(0, cfg.n_local, shared)
        srcs = []
        for i in range(cfg.n_sources):
            for j in range(sizes[1 + i]):
                put(1 + i, j, experts[cfg.n_local + i * per + j])
            srcs.append((st.buffers[1 + i].data_ptr(), i * per * st.rec, sizes[1 + i] * st.rec))
        dev.append(LayerWeights(torch.from_numpy(wr).to(DEV, adt),
                                None if b is None else torch.from_numpy(b).to(DEV), st.buffers[0], srcs))
        host.append(dict(experts=experts, shared=shared, wr=wr, b=b))
        stores.append(st)
    torch.cuda.synchronize()
    return host, dev, stores


@pytest.mark.parametrize("dt,engine,n_sets", [("f32", 0, 2), ("f32", 1, 2), ("bf16", 0, 2), ("bf16", 1, 2),
                                               ("bf16", 1, 3), ("f32", 0, 3)])
def test_pipeline_with_delays_matches_the_per_layer_oracle(dt, engine, n_sets):
    from split_weight_expert_amd import DWDPPipeline
    name, kw = CASES[dt]
    cfg = shrink(synth.get_config(name), **kw)
    host, layers, stores = build_layers(cfg)
    rec = stores[0].rec
    # small slices, so that a pull is many round-robin slices
    pipe = DWDPPipeline(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, cfg.n_local, DEV, slot_sets=n_sets,
                        chunk_bytes=max(4096, rec // 3 // 16 * 16), engine=engine, max_workgroups=3)
    adt = torch.float32 if dt == "f32" else torch.bfloat16
    x0 = torch.from_numpy(synth.tokens(cfg)).to(DEV, adt)
    for call in range(2):
        outs = [torch.empty(cfg.T, cfg.H, dtype=adt, device=DEV) for _ in range(L)]
        seen = {}

        def after(l, b):
            seen[l] = (b.logits.clone(), b.idx.clone())

        y = pipe.forward(x0, layers, outputs=outs, before_copy=lambda l: torch.cuda._sleep(SLEEP),
                         before_compute=lambda l: torch.cuda._sleep(SLEEP // 2), after_layer=after)
        torch.cuda.synchronize()
        assert y.data_ptr() == outs[-1].data_ptr()
        xin = x0
        for l in range(L):
            x_np = to_np(xin).astype(np.float32)
            lg = seen[l][0].cpu().numpy().astype(np.float64)
            gi = seen[l][1].cpu().numpy()
            np.testing.assert_array_equal(gi, omoe.topk_select(lg, cfg.k), err_msg=f"layer {l} routing")
            h = host[l]
            ref = omoe.moe_layer(x_np, h["wr"], h["b"], cfg.k, lambda e, h=h: h["experts"][e],
                                 (lambda h=h: h["shared"]) if cfg.shared else None, precision=dt,
                                 routing=(lg, gi, omoe.gate_weights(lg, gi)))
            assert_close(to_np(outs[l]), ref["y"], dt, f"call {call} layer {l} ({dt}, engine {engine}, {n_sets} sets)")
            xin = outs[l]
    del stores
