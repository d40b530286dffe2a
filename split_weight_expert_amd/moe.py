"""One DWDP rank's MoE block on top of the C ABI.

ExpertStore holds a layer's expert records in separate device buffers -- the
resident partition and a double-buffered prefetch area (DWDP paper summary,
§2) -- and builds the per-group pointer table that the grouped GEMM reads
instead of a merged copy (§4.2).  MoEBlock owns the activation buffers and
workspaces for a token count and runs route -> permute -> grouped FFN ->
combine on one stream.  By default GEMM1 reads the token rows through the
permutation (dwdp_moe_grouped_ffn_tokens) and no x_perm is materialised;
gather=True runs the permute's row gather and the x_perm path instead.
Nothing here computes: every step is a libdwdp call.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import api
from ._lib import BF16, F32, FP8_E4M3

DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}
_ACT_TORCH = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8}


def act_dtype(w_dtype: int) -> torch.dtype:
    """torch dtype of the tokens / block output (fp8 layers take bf16 tokens)."""
    return torch.float32 if w_dtype == F32 else torch.bfloat16


class ExpertStore:
    """Expert records of one layer in `n_buffers` separate device allocations.

    Buffer 0 is the resident partition; buffers 1.. are prefetch slot sets.
    A record is [W13 | W2 | S13 | S2] (include/dwdp.h), `rec` bytes long.
    """

    def __init__(self, H: int, I: int, w_dtype: int, slots_per_buffer, device="cuda"):
        self.H, self.I, self.w_dtype = H, I, w_dtype
        self.rec = api.expert_record_bytes(H, I, w_dtype)
        self.off_w2, self.off_s13, self.off_s2 = api.expert_record_offsets(H, I, w_dtype)
        self.buffers = [torch.empty(max(n, 1) * self.rec, dtype=torch.uint8, device=device) for n in slots_per_buffer]
        self.slots = list(slots_per_buffer)

    def record(self, buf: int, slot: int) -> torch.Tensor:
        assert 0 <= slot < self.slots[buf]
        return self.buffers[buf][slot * self.rec:(slot + 1) * self.rec]

    def record_ptr(self, buf: int, slot: int) -> int:
        return self.buffers[buf].data_ptr() + slot * self.rec

    def views(self, buf: int, slot: int):
        """(W13, W2, S13, S2) byte regions of one record (S* are None unless fp8).

        f32 weights are row-major; bf16 and fp8 weights are fragment-major (dwdp_pack_weights).
        """
        r = self.record(buf, slot)
        H, I = self.H, self.I
        eb = {F32: 4, BF16: 2, FP8_E4M3: 1}[self.w_dtype]
        w13 = r[:2 * I * H * eb]
        w2 = r[self.off_w2:self.off_w2 + H * I * eb]
        if self.w_dtype != FP8_E4M3:
            return w13, w2, None, None
        s13 = r[self.off_s13:self.off_s13 + (2 * I // 128) * (H // 128) * 4].view(torch.float32).view(2 * I // 128,
                                                                                                     H // 128)
        s2 = r[self.off_s2:self.off_s2 + (H // 128) * (I // 128) * 4].view(torch.float32).view(H // 128, I // 128)
        return w13, w2, s13, s2

    def load(self, buf: int, slot: int, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor, stream=None):
        """Place one expert's weights ([out, in] device tensors; fp32 masters for fp8) into a record."""
        w13, w2, s13, s2 = self.views(buf, slot)
        H, I = self.H, self.I
        if self.w_dtype == F32:
            w13.view(torch.float32).view(2 * I, H)[:I].copy_(wg)
            w13.view(torch.float32).view(2 * I, H)[I:].copy_(wu)
            w2.view(torch.float32).view(H, I).copy_(wd)
        elif self.w_dtype == BF16:
            api.pack_weights(torch.cat([wg, wu], 0).to(torch.bfloat16).contiguous(), w13, BF16, stream)
            api.pack_weights(wd.to(torch.bfloat16).contiguous(), w2, BF16, stream)
        else:
            q13 = torch.empty(2 * I, H, dtype=torch.uint8, device=w13.device)
            q2 = torch.empty(H, I, dtype=torch.uint8, device=w13.device)
            api.quantize_weight_fp8(torch.cat([wg, wu], 0).float().contiguous(), q13, s13, stream)
            api.quantize_weight_fp8(wd.float().contiguous(), q2, s2, stream)
            api.pack_weights(q13, w13, FP8_E4M3, stream)
            api.pack_weights(q2, w2, FP8_E4M3, stream)

    def check_placement(self, placement) -> None:
        """Every (buffer, slot) must name a record inside this store: the C ABI cannot check it, since it
        does not know the buffers' sizes, and the GEMM would read past the allocation."""
        for g, (buf, slot) in enumerate(placement):
            if not 0 <= buf < len(self.buffers):
                raise ValueError(f"group {g}: buffer {buf} is not one of the store's {len(self.buffers)} buffers")
            if not 0 <= slot < self.slots[buf]:
                raise ValueError(f"group {g}: slot {slot} is outside buffer {buf}'s {self.slots[buf]} records")

    def table(self, placement, device="cuda") -> torch.Tensor:
        """Device pointer table for placement = [(buffer, slot) for each group]."""
        self.check_placement(placement)
        t = api.fill_expert_table([b.data_ptr() for b in self.buffers], [p[0] for p in placement],
                                  [p[1] for p in placement], self.H, self.I, self.w_dtype)
        return api.table_to_device(t, device)


def dwdp_placement(E: int, n_local: int, shared: int, slot_set: int = 1):
    """Experts [0, n_local) and the shared expert resident (buffer 0); the rest in prefetch slot set `slot_set`."""
    pl = [(0, e) if e < n_local else (slot_set, e - n_local) for e in range(E)]
    if shared:
        pl.append((0, n_local))
    return pl


@dataclass
class BlockBuffers:
    logits: torch.Tensor
    idx: torch.Tensor
    w: torch.Tensor
    x_perm: torch.Tensor | None          # gather mode: permuted rows (fp8: codes)
    x_perm_scale: torch.Tensor | None    # gather mode, fp8
    x_q: torch.Tensor | None             # token mode, fp8: per-token codes [T, H]
    x_q_scale: torch.Tensor | None       # token mode, fp8: [T, H/128]
    offsets: torch.Tensor
    perm_src: torch.Tensor
    inv_perm: torch.Tensor
    y_perm: torch.Tensor
    y: torch.Tensor
    ws_perm: torch.Tensor
    ws_ffn: torch.Tensor
    x_tokens: torch.Tensor | None = None  # token mode: the rows GEMM1 reads (x, or x_q for fp8)


class MoEBlock:
    """Route -> permute -> grouped SwiGLU FFN -> combine for one layer shape."""

    def __init__(self, H: int, I: int, E: int, k: int, shared: int, dtype: str, device="cuda", gather: bool = False):
        self.H, self.I, self.E, self.k, self.shared = H, I, E, k, shared
        self.w_dtype = DTYPES[dtype]
        self.device = device
        self.gather = gather
        self._bufs: dict[int, BlockBuffers] = {}

    def buffers(self, T: int) -> BlockBuffers:
        if T in self._bufs:
            return self._bufs[T]
        H, I, E, k, S, dev = self.H, self.I, self.E, self.k, self.shared, self.device
        rows = T * k + S * T
        adt = act_dtype(self.w_dtype)
        xp_dt = torch.uint8 if self.w_dtype == FP8_E4M3 else adt
        fp8 = self.w_dtype == FP8_E4M3
        g = self.gather
        ws_p = api.workspace_bytes(api.OP_PERMUTE, T, k, E, H, I, self.w_dtype, S)
        ws_f = api.workspace_bytes(api.OP_GROUPED_FFN, T, k, E, H, I, self.w_dtype, S)
        b = BlockBuffers(
            logits=torch.empty(T, E, dtype=torch.float32, device=dev),
            idx=torch.empty(T, k, dtype=torch.int32, device=dev),
            w=torch.empty(T, k, dtype=torch.float32, device=dev),
            x_perm=torch.empty(rows, H, dtype=xp_dt, device=dev) if g else None,
            x_perm_scale=torch.empty(rows, H // 128, dtype=torch.float32, device=dev) if g and fp8 else None,
            x_q=torch.empty(T, H, dtype=torch.uint8, device=dev) if fp8 and not g else None,
            x_q_scale=torch.empty(T, H // 128, dtype=torch.float32, device=dev) if fp8 and not g else None,
            offsets=torch.empty(E + S + 1, dtype=torch.int32, device=dev),
            perm_src=torch.empty(rows, dtype=torch.int32, device=dev),
            inv_perm=torch.empty(T, k, dtype=torch.int32, device=dev),
            y_perm=torch.empty(rows, H, dtype=adt, device=dev),
            y=torch.empty(T, H, dtype=adt, device=dev),
            ws_perm=torch.empty(max(ws_p, 256), dtype=torch.uint8, device=dev),
            ws_ffn=torch.empty(max(ws_f, 256), dtype=torch.uint8, device=dev),
        )
        self._bufs[T] = b
        return b

    def route(self, x, w_router, bias, b: BlockBuffers, stream=None):
        api.route_topk(x, w_router, bias, self.k, b.logits, b.idx, b.w, stream)

    def permute(self, x, b: BlockBuffers, stream=None):
        """Expert permutation; gather mode also writes x_perm, token mode quantises the tokens for fp8."""
        fp8 = self.w_dtype == FP8_E4M3
        api.permute(b.idx, self.E, self.shared, x, self.w_dtype if fp8 else api.dtype_code(x),
                    b.x_perm, b.x_perm_scale, b.offsets, b.perm_src, b.inv_perm, b.ws_perm, stream)
        if not self.gather:
            if fp8:
                api.quantize_tokens_fp8(x, b.x_q, b.x_q_scale, stream)
                b.x_tokens = b.x_q
            else:
                b.x_tokens = x

    def ffn(self, table, b: BlockBuffers, stream=None):
        self.ffn_stage(0, table, b, stream)

    def ffn_stage(self, stage: int, table, b: BlockBuffers, stream=None):
        if self.gather:
            api.moe_grouped_ffn_stage(stage, table, self.E + self.shared, b.offsets, b.x_perm, b.x_perm_scale,
                                      self.H, self.I, self.w_dtype, b.y_perm, b.ws_ffn, stream)
        else:
            api.moe_grouped_ffn_tokens(stage, table, self.E + self.shared, b.offsets, b.perm_src, b.x_tokens,
                                       b.x_q_scale, self.H, self.I, self.w_dtype, b.y_perm, b.ws_ffn, stream)

    def combine(self, b: BlockBuffers, stream=None, out=None):
        api.combine(b.y_perm, b.inv_perm, b.w, self.shared, b.y if out is None else out, stream)

    def forward(self, x, w_router, bias, table, stream=None, out=None) -> BlockBuffers:
        """The whole block on `stream`; results stay in the returned buffers (y in `out` if given)."""
        b = self.buffers(x.shape[0])
        self.route(x, w_router, bias, b, stream)
        self.permute(x, b, stream)
        self.ffn(table, b, stream)
        self.combine(b, stream, out)
        return b


@dataclass
class LayerWeights:
    """One MoE layer in the DWDP layout of a rank.

    resident: the rank's own records of the layer, experts [0, n_local) then the shared expert, in
    one device buffer (the resident partition, DWDP paper summary §2).  sources: where the layer's
    other E - n_local expert records are pulled from, as (device pointer, offset in the slot set,
    bytes) -- on one GPU, separate device allocations stand in for the peers' HBM; record e sits at
    offset (e - n_local) * record_bytes of the slot set.
    """
    w_router: torch.Tensor
    bias: torch.Tensor | None
    resident: torch.Tensor
    sources: list


class DWDPPipeline:
    """Layer-ahead prefetch over a ring of N >= 2 prefetch slot sets (DWDP paper summary §2, §4.3.2).

    With the pages' double buffer (N = 2), while layer l computes on the compute stream from slot set
    l % 2, a copy stream pulls layer l+1's non-local experts into slot set (l + 1) % 2 in fixed-size
    slices, round-robin over the sources.  With N slot sets the pull of layer l + N - 1 starts as soon
    as layer l - 1 has released its slot set, so each pull may spread over N - 1 layers of compute
    (one GPU's 288 GB of HBM holds several fp8 slot sets of a DeepSeek-R1 layer, 8.5 GB each).  Two
    hazards are ordered with events: layer l waits for the copy that filled its slot set, and a copy
    into a slot set waits for the layer that last read it.  The layer time is then max(compute,
    copy / (N - 1)) (the layer-wise model of the pages, §3, for N = 2), not their sum.

    The block reads each layer's weights through a pointer table over two buffers -- the layer's
    resident records and the current slot set -- so nothing is merged.  Only the MoE blocks run here
    (a model without attention): layer l+1's input is layer l's output.
    """

    def __init__(self, H: int, I: int, E: int, k: int, shared: int, dtype: str, n_local: int, device="cuda",
                 slot_sets=None, chunk_bytes: int = 4 << 20, engine: int = api.COPY_KERNEL,
                 max_workgroups: int = 48):
        self.H, self.I, self.E, self.k, self.shared, self.n_local = H, I, E, k, shared, n_local
        self.w_dtype = DTYPES[dtype]
        self.device = torch.device(device)
        self.rec = api.expert_record_bytes(H, I, self.w_dtype)
        self.n_pre = E - n_local
        if slot_sets is None or isinstance(slot_sets, int):
            n = 2 if slot_sets is None else slot_sets
            slot_sets = [torch.empty(max(self.n_pre, 1) * self.rec, dtype=torch.uint8, device=self.device)
                         for _ in range(n)]
        assert len(slot_sets) >= 2 and all(t.numel() >= self.n_pre * self.rec for t in slot_sets)
        self.slot_sets = list(slot_sets)
        self.chunk_bytes, self.engine, self.max_workgroups = chunk_bytes, engine, max_workgroups
        self.block = MoEBlock(H, I, E, k, shared, dtype, self.device)
        self.copy_stream = torch.cuda.Stream(self.device)
        self._last_read = [None] * len(self.slot_sets)   # event of the last layer that read each slot set
        self._tables = {}

    def placement(self):
        """(buffer, slot) of every group: 0 = the layer's resident records, 1 = the current slot set."""
        pl = [(0, e) if e < self.n_local else (1, e - self.n_local) for e in range(self.E)]
        if self.shared:
            pl.append((0, self.n_local))
        return pl

    def table(self, layer: LayerWeights, s: int) -> torch.Tensor:
        key = (layer.resident.data_ptr(), s)
        if key not in self._tables:
            assert layer.resident.numel() >= (self.n_local + self.shared) * self.rec, "resident buffer too small"
            pl = self.placement()
            t = api.fill_expert_table([layer.resident.data_ptr(), self.slot_sets[s].data_ptr()],
                                      [p[0] for p in pl], [p[1] for p in pl], self.H, self.I, self.w_dtype)
            self._tables[key] = api.table_to_device(t, self.device)
        return self._tables[key]

    def check_sources(self, layer: LayerWeights):
        for _, off, n in layer.sources:
            assert 0 <= off and off + n <= self.n_pre * self.rec, "a source lands outside the slot set"

    def prefetch(self, layer: LayerWeights, s: int, wait=None, done=None):
        """Enqueue the pull of `layer`'s non-local records into slot set s on the copy stream."""
        api.prefetch_chunks(self.slot_sets[s].data_ptr(), layer.sources, self.chunk_bytes, engine=self.engine,
                            max_workgroups=self.max_workgroups, copy_stream=self.copy_stream, wait_event=wait,
                            done_event=done)

    def forward(self, x: torch.Tensor, layers, outputs=None, before_copy=None, before_compute=None,
                after_layer=None, chain: bool = True) -> torch.Tensor:
        """Run the layers in order on the current stream, each on the previous one's output (or, with
        chain=False, every layer on x: a benchmark of layers with a fixed input distribution).

        outputs: optional list of L [T, H] tensors that receive every layer's output (else two
        alternating buffers are used and only the last output is returned).  The hooks are called at
        enqueue time: before_copy(l) with the copy stream current, before layer l's pull is enqueued;
        before_compute(l) and after_layer(l, block_buffers) with the compute stream current, around
        layer l's block.  Returns the last layer's output.
        """
        comp = torch.cuda.current_stream(self.device)
        L = len(layers)
        for lw in layers:
            self.check_sources(lw)
        T = x.shape[0]
        if outputs is None:
            bufs = [torch.empty(T, self.H, dtype=x.dtype, device=self.device) for _ in range(min(L, 2))]
            outputs = [bufs[l % 2] for l in range(L)]
        N = len(self.slot_sets)
        copy_done = [torch.cuda.Event() for _ in range(N)]
        # the copy stream must not start before everything already enqueued on the compute stream
        # that produced the sources or this call's input
        start = torch.cuda.Event()
        start.record(comp)
        self.copy_stream.wait_event(start)

        def pull(l, s):
            with torch.cuda.stream(self.copy_stream):
                if before_copy is not None:
                    before_copy(l)
            self.prefetch(layers[l], s, wait=self._last_read[s], done=copy_done[s])

        # layers 0 .. N-2 into slot sets 0 .. N-2 (each waits for its set's last reader of an earlier call)
        for l in range(min(L, N - 1)):
            pull(l, l)
        for l in range(L):
            s = l % N
            comp.wait_event(copy_done[s])
            if before_compute is not None:
                before_compute(l)
            lw = layers[l]
            b = self.block.forward(x, lw.w_router, lw.bias, self.table(lw, s), out=outputs[l])
            if after_layer is not None:
                after_layer(l, b)
            ev = torch.cuda.Event()
            ev.record(comp)
            # the pull into slot set (l - 1) % N, released by layer l - 1 (or by an earlier call), is
            # enqueued after layer l's block: an engine whose enqueue blocks the host (the DMA engines
            # when their queue is full) then does not hold back the block's launches
            if l + N - 1 < L:
                pull(l + N - 1, (l + N - 1) % N)
            self._last_read[s] = ev
            if chain:
                x = outputs[l]
        return outputs[L - 1] if L else x
