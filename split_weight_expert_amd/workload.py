"""A synthetic MoE layer resident on the GPU in the DWDP layout.

Benchmark and test helper: allocates the expert store -- one resident buffer
(experts [0, n_local) and the shared expert), two prefetch slot sets, and
optionally separate source regions standing in for the peers' HBM -- and
fills it from the seeded generator directly on the device.  The compute path
(MoEBlock) does not depend on this module.
"""
from __future__ import annotations

import torch

import synth
from synth import gen

from .moe import DTYPES, ExpertStore, MoEBlock, act_dtype, dwdp_placement


def _fill(key, n, std, kind, ptr, stream):
    gen.gpu_fill(key, n, std, kind, ptr, stream.cuda_stream)


class DeviceLayer:
    """Tokens, router and expert records of one synthetic layer (and optionally the next layer's sources)."""

    def __init__(self, cfg: synth.LayerConfig, device="cuda", layer: int = 0, sources: bool = False,
                 slot_sets: int = 2, T: int | None = None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.layer = layer
        self.w_dtype = DTYPES[cfg.dtype]
        H, I, E = cfg.H, cfg.I, cfg.E
        self.T = cfg.T if T is None else T
        st = torch.cuda.current_stream(self.device)
        adt = act_dtype(self.w_dtype)
        tk = gen.token_kind(cfg)
        self.x = torch.empty(self.T, H, dtype=adt, device=self.device)
        _fill(gen.tokens_key(cfg, layer), self.T * H, 1.0, tk, self.x.data_ptr(), st)
        self.w_router = torch.from_numpy(synth.router_weight(cfg, layer)).to(self.device, adt)
        b = synth.router_bias(cfg, layer)
        self.bias = None if b is None else torch.from_numpy(b).to(self.device)
        n_pre = cfg.n_prefetch
        slots = [cfg.n_local + cfg.shared] + [n_pre] * slot_sets
        self.store = ExpertStore(H, I, self.w_dtype, slots, device=self.device)
        for e in range(cfg.n_local):
            self.fill_record(self.store, 0, e, e, layer)
        if cfg.shared:
            self.fill_record(self.store, 0, cfg.n_local, E, layer)
        for e in range(cfg.n_local, E):
            self.fill_record(self.store, 1, e - cfg.n_local, e, layer)
        self.sources = None
        if sources:
            # the next layer's non-local experts, split evenly over the stand-in source regions
            per = n_pre // cfg.n_sources
            assert per * cfg.n_sources == n_pre
            self.src_store = ExpertStore(H, I, self.w_dtype, [per] * cfg.n_sources, device=self.device)
            for s in range(cfg.n_sources):
                for i in range(per):
                    self.fill_record(self.src_store, s, i, cfg.n_local + s * per + i, layer + 1)
            self.sources = [(self.src_store.buffers[s].data_ptr(), s * per * self.store.rec, per * self.store.rec)
                            for s in range(cfg.n_sources)]
        torch.cuda.synchronize(self.device)

    def fill_record(self, store: ExpertStore, buf: int, slot: int, expert: int, layer: int):
        """Write expert `expert` of layer `layer` (E = the shared expert) into store record (buf, slot)."""
        cfg = self.cfg
        H, I = cfg.H, cfg.I
        kg, ku, kd = gen.expert_keys(cfg, expert, layer)
        sg, su, sd = gen.expert_stds(cfg)
        st = torch.cuda.current_stream(self.device)
        kind = gen.expert_kind(cfg)
        dt = torch.float32 if kind == "f32" else torch.bfloat16
        w13 = torch.empty(2 * I, H, dtype=dt, device=self.device)
        wd = torch.empty(H, I, dtype=dt, device=self.device)
        _fill(kg, I * H, sg, kind, w13.data_ptr(), st)
        _fill(ku, I * H, su, kind, w13.data_ptr() + I * H * w13.element_size(), st)
        _fill(kd, H * I, sd, kind, wd.data_ptr(), st)
        store.load(buf, slot, w13[:I], w13[I:], wd)

    def table(self, slot_set: int = 1) -> torch.Tensor:
        c = self.cfg
        return self.store.table(dwdp_placement(c.E, c.n_local, c.shared, slot_set), self.device)

    def block(self) -> MoEBlock:
        c = self.cfg
        return MoEBlock(c.H, c.I, c.E, c.k, c.shared, c.dtype, self.device)
