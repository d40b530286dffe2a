"""ctypes loader for libdwdp.so, the C ABI declared in include/dwdp.h.

The library is the only compute path: if it is not built, importing this
module raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DWDP_LIBRARY may name another build of the same library (e.g. one compiled with different tile settings)
LIB_PATH = os.environ.get("DWDP_LIBRARY") or os.path.join(HERE, "lib", "libdwdp.so")

DWDP_OK, DWDP_ERR_INVALID_ARG, DWDP_ERR_UNSUPPORTED, DWDP_ERR_WORKSPACE, DWDP_ERR_HIP = range(5)
F32, BF16, FP8_E4M3 = 0, 1, 2
OP_PERMUTE, OP_GROUPED_FFN = 0, 1
COPY_HIPMEMCPY, COPY_KERNEL, COPY_SDMA = 0, 1, 2


class ExpertPtrs(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("s13", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class CopySrc(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst_offset", ctypes.c_size_t), ("bytes", ctypes.c_size_t)]


class Chunk(ctypes.Structure):
    _fields_ = [("source", ctypes.c_int32), ("pad_", ctypes.c_int32), ("src_offset", ctypes.c_size_t),
                ("dst_offset", ctypes.c_size_t), ("bytes", ctypes.c_size_t)]


class TileRecord(ctypes.Structure):
    _fields_ = [("t_start", ctypes.c_uint64), ("t_end", ctypes.c_uint64), ("order", ctypes.c_int32),
                ("group", ctypes.c_int32), ("first_row", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("n_tile", ctypes.c_int32), ("group_m_tiles", ctypes.c_int32), ("xcd", ctypes.c_int32),
                ("hw_id", ctypes.c_int32)]


class DwdpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dwdp error {code}: {msg}")
        self.code = code


# name -> (restype, argtypes)
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "dwdp_route_topk": (_i32, [_vp, _vp, _i32, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "dwdp_permute": (_i32, [_vp, _i64, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                            _vp]),
    "dwdp_moe_grouped_ffn": (_i32, [_vp, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "dwdp_moe_grouped_ffn_stage": (_i32, [_i32, _vp, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _sz,
                                          _vp]),
    "dwdp_moe_grouped_ffn_tokens": (_i32, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp,
                                           _vp, _sz, _vp]),
    "dwdp_moe_grouped_ffn_tokens_static": (_i32, [_i32, _vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32,
                                                  _vp, _vp]),
    "dwdp_static_scratch_bytes": (_sz, []),
    "dwdp_quantize_tokens_fp8": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "dwdp_combine": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp]),
    "dwdp_prefetch_chunks": (_i32, [_vp, _vp, _i32, _sz, _i32, _i32, _vp, _vp, _vp]),
    "dwdp_prefetch_plan": (_i32, [_vp, _i32, _sz, _vp, _sz, ctypes.POINTER(_sz)]),
    "dwdp_fill_expert_table": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "dwdp_expert_record_bytes": (_sz, [_i32, _i32, _i32]),
    "dwdp_expert_record_offsets": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                          ctypes.POINTER(_sz)]),
    "dwdp_pack_weights": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "dwdp_quantize_weight_fp8": (_i32, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "dwdp_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32]),
    "dwdp_diag_operand_stream": (_i32, [_vp, _sz, _sz, _i32, _i32, _i32, _i32, _vp]),
    "dwdp_diag_lds_read": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp]),
    "dwdp_diag_tile_trace_clear": (_i32, [_vp]),
    "dwdp_diag_tile_trace_read": (_i32, [_vp, _sz, ctypes.POINTER(_sz)]),
    "dwdp_last_error": (ctypes.c_char_p, []),
    "dwdp_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libdwdp.so and attach the C signatures; raises if it is not built."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime (same soname, libamdhip64.so.7).  Loading it first makes this
        # library bind to that same runtime instance; a second HIP runtime in the process cannot open
        # the GPU once torch's has.
        import torch  # noqa: F401
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built (run __graft_entry__.build()); there is no fallback path")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(rc: int) -> None:
    if rc != DWDP_OK:
        raise DwdpError(rc, load().dwdp_last_error().decode())
