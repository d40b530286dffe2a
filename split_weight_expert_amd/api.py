"""Thin Python binding of the C ABI (same names, argument marshalling only).

torch tensors supply device memory and streams; every step of the MoE block
runs in libdwdp.so's HIP kernels.  Shapes and dtypes follow include/dwdp.h.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import BF16, COPY_HIPMEMCPY, COPY_KERNEL, COPY_SDMA, F32, FP8_E4M3, OP_GROUPED_FFN, OP_PERMUTE  # noqa: F401

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.uint8: FP8_E4M3}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _event(ev, stream=None):
    """hipEvent_t of a torch event; torch creates events lazily, so an unrecorded one is first recorded."""
    if ev is None:
        return None
    if ev.cuda_event == 0:
        ev.record(torch.cuda.current_stream() if stream is None else stream)
    return ctypes.c_void_p(ev.cuda_event)


def dtype_code(t: torch.Tensor) -> int:
    return _DT[t.dtype]


def version() -> str:
    return _lib.load().dwdp_version().decode()


def workspace_bytes(op: int, T: int, k: int, E: int, H: int, I: int, dtype: int, shared: int) -> int:
    return int(_lib.load().dwdp_workspace_bytes(op, T, k, E, H, I, dtype, shared))


def route_topk(x, w_router, bias, k, logits_out, topk_idx, topk_w, stream=None):
    T, H = x.shape
    E = w_router.shape[0]
    _lib.check(_lib.load().dwdp_route_topk(_ptr(x), _ptr(w_router), dtype_code(x), _ptr(bias), T, H, E, k,
                                           _ptr(logits_out), _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def permute(topk_idx, E, shared, x, act_dtype, x_perm, x_perm_scale, offsets, perm_src, inv_perm, ws,
            stream=None):
    T, k = topk_idx.shape
    H = x.shape[1]
    _lib.check(_lib.load().dwdp_permute(_ptr(topk_idx), T, k, E, shared, _ptr(x), dtype_code(x), act_dtype, H,
                                        _ptr(x_perm), _ptr(x_perm_scale), _ptr(offsets), _ptr(perm_src),
                                        _ptr(inv_perm), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                        _stream(stream)))


def moe_grouped_ffn(table, n_groups, offsets, x_perm, x_perm_scale, H, I, w_dtype, y_perm, ws, stream=None):
    rows = x_perm.shape[0]
    _lib.check(_lib.load().dwdp_moe_grouped_ffn(_ptr(table), n_groups, _ptr(offsets), _ptr(x_perm),
                                                _ptr(x_perm_scale), rows, H, I, w_dtype, _ptr(y_perm), _ptr(ws),
                                                0 if ws is None else ws.numel() * ws.element_size(),
                                                _stream(stream)))


def moe_grouped_ffn_stage(stage, table, n_groups, offsets, x_perm, x_perm_scale, H, I, w_dtype, y_perm, ws,
                          stream=None):
    rows = x_perm.shape[0]
    _lib.check(_lib.load().dwdp_moe_grouped_ffn_stage(stage, _ptr(table), n_groups, _ptr(offsets), _ptr(x_perm),
                                                      _ptr(x_perm_scale), rows, H, I, w_dtype, _ptr(y_perm),
                                                      _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                                      _stream(stream)))


def moe_grouped_ffn_tokens(stage, table, n_groups, offsets, perm_src, x, x_scale, H, I, w_dtype, y_perm, ws,
                           stream=None):
    """Grouped FFN whose GEMM1 reads token rows x[perm_src[r]] (no x_perm)."""
    rows = perm_src.shape[0]
    T = x.shape[0]
    _lib.check(_lib.load().dwdp_moe_grouped_ffn_tokens(stage, _ptr(table), n_groups, _ptr(offsets), _ptr(perm_src),
                                                       _ptr(x), _ptr(x_scale), T, rows, H, I, w_dtype, _ptr(y_perm),
                                                       _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                                       _stream(stream)))


def moe_grouped_ffn_tokens_static(stage, table, n_groups, offsets, perm_src, x, x_scale, H, I, w_dtype, y_perm,
                                  stream=None):
    """moe_grouped_ffn_tokens with the library's fixed workspace array (no workspace argument)."""
    rows = perm_src.shape[0]
    T = x.shape[0]
    _lib.check(_lib.load().dwdp_moe_grouped_ffn_tokens_static(stage, _ptr(table), n_groups, _ptr(offsets),
                                                              _ptr(perm_src), _ptr(x), _ptr(x_scale), T, rows, H, I,
                                                              w_dtype, _ptr(y_perm), _stream(stream)))


def static_scratch_bytes() -> int:
    return int(_lib.load().dwdp_static_scratch_bytes())


def quantize_tokens_fp8(x, q, q_scale, stream=None):
    T, H = x.shape
    _lib.check(_lib.load().dwdp_quantize_tokens_fp8(_ptr(x), T, H, _ptr(q), _ptr(q_scale), _stream(stream)))


def combine(y_perm, inv_perm, topk_w, shared, y, stream=None):
    T, k = inv_perm.shape
    H = y.shape[1]
    _lib.check(_lib.load().dwdp_combine(_ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), T, k, shared, H, dtype_code(y),
                                        _ptr(y), _stream(stream)))


def _sources(srcs):
    """srcs: list of (device pointer int, dst_offset, bytes)."""
    arr = (_lib.CopySrc * len(srcs))()
    for i, (p, off, n) in enumerate(srcs):
        arr[i].src = p
        arr[i].dst_offset = off
        arr[i].bytes = n
    return arr


def prefetch_chunks(dst_ptr, srcs, chunk_bytes, engine=COPY_KERNEL, max_workgroups=0, copy_stream=None,
                    wait_event=None, done_event=None):
    arr = _sources(srcs)
    _lib.check(_lib.load().dwdp_prefetch_chunks(ctypes.c_void_p(dst_ptr), arr, len(srcs), chunk_bytes, engine,
                                                max_workgroups, _stream(copy_stream), _event(wait_event),
                                                _event(done_event, copy_stream)))


def prefetch_plan(srcs, chunk_bytes):
    """Host-only: the slice plan as a list of (source, src_offset, dst_offset, bytes)."""
    arr = _sources(srcs)
    n = ctypes.c_size_t(0)
    lib = _lib.load()
    _lib.check(lib.dwdp_prefetch_plan(arr, len(srcs), chunk_bytes, None, 0, ctypes.byref(n)))
    out = (_lib.Chunk * max(n.value, 1))()
    _lib.check(lib.dwdp_prefetch_plan(arr, len(srcs), chunk_bytes, out, n.value, ctypes.byref(n)))
    return [(c.source, c.src_offset, c.dst_offset, c.bytes) for c in out[:n.value]]


def expert_record_bytes(H, I, w_dtype) -> int:
    return int(_lib.load().dwdp_expert_record_bytes(H, I, w_dtype))


def expert_record_offsets(H, I, w_dtype):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(_lib.load().dwdp_expert_record_offsets(H, I, w_dtype, ctypes.byref(a), ctypes.byref(b),
                                                      ctypes.byref(c)))
    return a.value, b.value, c.value


def fill_expert_table(buffer_ptrs, buf_of, slot_of, H, I, w_dtype):
    """Host-only: the pointer table for a placement, as a ctypes array of ExpertPtrs."""
    n = len(buf_of)
    bufs = (ctypes.c_void_p * len(buffer_ptrs))(*buffer_ptrs)
    bo = (ctypes.c_int32 * n)(*buf_of)
    so = (ctypes.c_int32 * n)(*slot_of)
    out = (_lib.ExpertPtrs * n)()
    _lib.check(_lib.load().dwdp_fill_expert_table(bufs, len(buffer_ptrs), bo, so, n, H, I, w_dtype, out))
    return out


def table_to_device(table, device) -> torch.Tensor:
    """Upload a host pointer table to device memory (uint8 tensor of 32 bytes per group)."""
    raw = torch.frombuffer(bytearray(bytes(table)), dtype=torch.uint8)
    return raw.to(device)


def quantize_weight_fp8(w, q, s, stream=None):
    rows, cols = w.shape
    _lib.check(_lib.load().dwdp_quantize_weight_fp8(_ptr(w), rows, cols, _ptr(q), _ptr(s), _stream(stream)))


def pack_weights(w, out, dtype_code_, stream=None):
    """Re-lay a weight matrix w [N, K] (bf16, or uint8 E4M3 codes) into the fragment-major layout in out."""
    N, K = w.shape
    _lib.check(_lib.load().dwdp_pack_weights(_ptr(w), N, K, dtype_code_, _ptr(out), _stream(stream)))


# ------------------------------------------------------------------ diagnostics (not steps of the block)

def diag_operand_stream(src, span, stride, iters, grid, in_flight=3, cpol=0, stream=None):
    """Operand-stream probe over the uint8 device tensor src: grid workgroups each read span bytes at
    b*stride, iters times, into an LDS ring with in_flight 32 KB steps outstanding."""
    need = (grid - 1) * stride + span
    if src.dtype != torch.uint8 or not src.is_cuda or src.numel() < need:
        raise ValueError(f"src must be a uint8 device tensor of at least {need} bytes")
    _lib.check(_lib.load().dwdp_diag_operand_stream(_ptr(src), span, stride, iters, grid, in_flight, cpol,
                                                    _stream(stream)))


def diag_lds_read(grid, waves, iters, stream=None):
    """LDS read probe; returns (bytes per shader clock per CU, shader-clock GHz) averaged over the
    workgroups (synchronises the stream)."""
    import numpy as np
    dev = torch.device("cuda", torch.cuda.current_device())
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    clocks = torch.zeros(2 * grid, dtype=torch.int64, device=dev)
    _lib.check(_lib.load().dwdp_diag_lds_read(grid, waves, iters, _ptr(sink), _ptr(clocks), _stream(stream)))
    (stream or torch.cuda.current_stream()).synchronize()
    c = clocks.cpu().numpy().astype(np.float64).reshape(grid, 2)
    nbytes = float(iters) * 16384 * waves
    return float(np.mean(nbytes / c[:, 0])), float(np.mean(c[:, 0] / (c[:, 1] * 10.0)))


def diag_tile_trace_clear(stream=None):
    _lib.check(_lib.load().dwdp_diag_tile_trace_clear(_stream(stream)))


def diag_tile_trace_read(max_records=1 << 17):
    """Tile records of the last expert-GEMM launch as a numpy structured array (tile-trace builds)."""
    import numpy as np
    buf = (_lib.TileRecord * max_records)()
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().dwdp_diag_tile_trace_read(buf, max_records, ctypes.byref(n)))
    dt = np.dtype([("t_start", "<u8"), ("t_end", "<u8"), ("order", "<i4"), ("group", "<i4"), ("first_row", "<i4"),
                   ("rows", "<i4"), ("n_tile", "<i4"), ("group_m_tiles", "<i4"), ("xcd", "<i4"),
                   ("hw_id", "<i4")])
    assert dt.itemsize == ctypes.sizeof(_lib.TileRecord)
    return np.frombuffer(bytes(buf)[: n.value * dt.itemsize], dtype=dt).copy()
