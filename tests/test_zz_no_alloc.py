"""The no-allocation grouped FFN (dwdp_moe_grouped_ffn_tokens_static) against the workspace entry point.

The static variant keeps the grouped FFN's workspace in a fixed 64 MiB device array of the library
instead of a caller-provided buffer.  Through the C ABI, two calls in a row -- the second with fewer
tokens, so it runs over what the first left in the array -- must give bitwise the y_perm (and, after
stage 1, the A) of dwdp_moe_grouped_ffn_tokens with a freshly allocated workspace, for f32, bf16 and
fp8 weights; a shape whose workspace exceeds the array is rejected before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from synth.configs import shrink
from tests.gpu_util import HostLayer, need_gpu, upload_layer

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "f32": ("tiny_f32", dict(T=200, H=256, I=128, E=8, k=2, shared=1, n_local=4)),
    "bf16": ("prefill8k_bf16", dict(T=300, H=512, I=256, E=8, k=2, n_local=4)),
    "fp8": ("prefill16k_fp8", dict(T=300, H=512, I=256, E=8, k=2, n_local=4)),
}


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run_both(cfg, h, T):
    """Route and permute the first T tokens, then the grouped FFN through both entry points."""
    from split_weight_expert_amd import MoEBlock, api
    from split_weight_expert_amd._lib import DWDP_OK, load
    pl = [(0, e) if e < cfg.n_local else (1, e - cfg.n_local) for e in range(cfg.E)]
    slots = [cfg.n_local + cfg.shared, cfg.E - cfg.n_local]
    if cfg.shared:
        pl.append((0, cfg.n_local))
    store, table, x, wr, b = upload_layer(h, pl, slots)
    x = x[:T].contiguous()
    blk = MoEBlock(cfg.H, cfg.I, cfg.E, cfg.k, cfg.shared, cfg.dtype, DEV)
    bb = blk.buffers(T)
    blk.route(x, wr, b, bb)
    blk.permute(x, bb)
    G = cfg.E + cfg.shared
    rows = T * (cfg.k + cfg.shared)
    assert api.workspace_bytes(api.OP_GROUPED_FFN, T, cfg.k, cfg.E, cfg.H, cfg.I, blk.w_dtype, cfg.shared) \
        <= api.static_scratch_bytes()
    # reference: the workspace entry point, stage by stage
    api.moe_grouped_ffn_tokens(1, table, G, bb.offsets, bb.perm_src, bb.x_tokens, bb.x_q_scale, cfg.H, cfg.I,
                               blk.w_dtype, None, bb.ws_ffn)
    ea = {0: 4, 1: 2, 2: 1}[blk.w_dtype]
    a_ref = bb.ws_ffn[:rows * cfg.I * ea].clone()
    api.moe_grouped_ffn_tokens(2, table, G, bb.offsets, bb.perm_src, bb.x_tokens, bb.x_q_scale, cfg.H, cfg.I,
                               blk.w_dtype, bb.y_perm, bb.ws_ffn)
    y_ref = bb.y_perm.clone()
    # the static variant, through the C ABI directly: both stages in one call ...
    lib = load()
    y0 = torch.full_like(bb.y_perm, 7)
    sc = ctypes.c_void_p(0 if bb.x_q_scale is None else bb.x_q_scale.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.dwdp_moe_grouped_ffn_tokens_static(0, ctypes.c_void_p(table.data_ptr()), G,
                                                ctypes.c_void_p(bb.offsets.data_ptr()),
                                                ctypes.c_void_p(bb.perm_src.data_ptr()),
                                                ctypes.c_void_p(bb.x_tokens.data_ptr()), sc, T, rows, cfg.H, cfg.I,
                                                blk.w_dtype, ctypes.c_void_p(y0.data_ptr()), st)
    assert rc == DWDP_OK, lib.dwdp_last_error()
    # ... and stage 1 then stage 2 (stage 2 reads the A that stage 1 left in the array)
    y1 = torch.full_like(bb.y_perm, 9)
    api.moe_grouped_ffn_tokens_static(1, table, G, bb.offsets, bb.perm_src, bb.x_tokens, bb.x_q_scale, cfg.H, cfg.I,
                                      blk.w_dtype, None)
    api.moe_grouped_ffn_tokens_static(2, table, G, bb.offsets, bb.perm_src, bb.x_tokens, bb.x_q_scale, cfg.H, cfg.I,
                                      blk.w_dtype, y1)
    torch.cuda.synchronize()
    del store
    return a_ref, y_ref, y0, y1


@pytest.mark.parametrize("dt", ["f32", "bf16", "fp8"])
def test_static_workspace_variant_matches_the_workspace_entry_point(dt):
    name, kw = CASES[dt]
    cfg = shrink(synth.get_config(name), **kw)
    h = HostLayer(cfg)
    for T in (cfg.T, cfg.T // 3):            # the second call is smaller and runs over the first one's leftovers
        _, y_ref, y0, y1 = run_both(cfg, h, T)
        assert torch.equal(y0.view(torch.uint8), y_ref.view(torch.uint8)), f"{dt} T={T}: one-call static variant"
        assert torch.equal(y1.view(torch.uint8), y_ref.view(torch.uint8)), f"{dt} T={T}: staged static variant"


def test_static_workspace_variant_rejects_shapes_beyond_its_array():
    from split_weight_expert_amd import api
    from split_weight_expert_amd._lib import DWDP_ERR_WORKSPACE, load
    lib = load()
    cap = api.static_scratch_bytes()
    assert cap == 64 << 20
    # 8192 tokens of the 7168 x 2048 bf16 layer need a 302 MB A: rejected, nothing launched (null pointers)
    T, k, E, H, I = 8192, 8, 256, 7168, 2048
    rows = T * (k + 1)
    assert api.workspace_bytes(api.OP_GROUPED_FFN, T, k, E, H, I, api.BF16, 1) > cap
    rc = lib.dwdp_moe_grouped_ffn_tokens_static(0, None, E + 1, None, None, None, None, T, rows, H, I, api.BF16,
                                                None, None)
    assert rc == DWDP_ERR_WORKSPACE and b"static scratch" in lib.dwdp_last_error()
