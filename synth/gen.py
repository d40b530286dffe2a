"""Seeded element generator (host C and GPU HIP) and the layer-level synthetic tensors.

Distributions: tokens ~ N(0, 1); router and expert weights ~ N(0, 1/fan_in)
with fan_in = H for the router, gate and up projections and fan_in = I for the
down projection; the optional router-logit bias is N(0, 0.5) per expert
(0.5 read as the variance) or a Zipf(s = 1.1) log-popularity over a seeded
permutation of the experts.  The normal variates are the Irwin-Hall (n = 4)
approximation described in synth_host.c, which both implementations can
reproduce bit for bit.  bf16 workloads round every generated value to bf16
(round to nearest even) inside the generator; fp8 workloads keep the expert
weights as fp32 master values that each side block-quantises on its own.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

from .configs import LayerConfig

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15

TENSOR_X, TENSOR_ROUTER, TENSOR_BIAS, TENSOR_WG, TENSOR_WU, TENSOR_WD = range(6)

SEED = 0
_IH_SIGMA = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")


def _mix64(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def tensor_key(*ids: int) -> int:
    """64-bit key of the tensor named by the id tuple (seed, workload, layer, tensor, expert)."""
    h = 0x6A09E667F3BCC908
    for v in ids:
        h = _mix64((h ^ (int(v) & M64)) + GAMMA)
    return h


def scale_const(std: float) -> np.float32:
    """fp32 multiplier that turns a centred Irwin-Hall sum into a variate of deviation `std`."""
    return np.float32(std / _IH_SIGMA)


_host = None
_gpu = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, f32 = ctypes.c_uint64, ctypes.c_float
        for name in ("synth_fill_f32", "synth_fill_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, f32, ctypes.c_void_p]
            fn.restype = None
        lib.synth_gather_f32.argtypes = [u64, ctypes.c_void_p, u64, f32, ctypes.c_void_p]
        lib.synth_gather_f32.restype = None
        _host = lib
    return _host


def _gpu_lib():
    global _gpu
    if _gpu is None:
        import torch  # noqa: F401  -- bind to torch's HIP runtime instance (see split_weight_expert_amd._lib)
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        u64, f32, vp = ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
        for name in ("synth_gpu_fill_f32", "synth_gpu_fill_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, f32, vp, vp]
            fn.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def host_fill(key: int, n: int, std: float, kind: str, first: int = 0) -> np.ndarray:
    """Elements [first, first+n) of the tensor with `key`: float32, or uint16 bf16 bits for kind 'bf16'."""
    c = scale_const(std)
    lib = _host_lib()
    if kind == "f32":
        out = np.empty(n, np.float32)
        lib.synth_fill_f32(key, first, n, c, out.ctypes.data)
    elif kind == "bf16":
        out = np.empty(n, np.uint16)
        lib.synth_fill_bf16(key, first, n, c, out.ctypes.data)
    else:
        raise ValueError(kind)
    return out


def host_gather(key: int, idx: np.ndarray, std: float) -> np.ndarray:
    """fp32 elements idx[j] of the tensor with `key` (sampling a large tensor)."""
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.shape, np.float32)
    _host_lib().synth_gather_f32(key, idx.ctypes.data, idx.size, scale_const(std), out.ctypes.data)
    return out


def gpu_fill(key: int, n: int, std: float, kind: str, out_ptr: int, stream: int = 0, first: int = 0) -> None:
    """Write elements [first, first+n) of the tensor with `key` to device memory at out_ptr."""
    lib = _gpu_lib()
    fn = {"f32": lib.synth_gpu_fill_f32, "bf16": lib.synth_gpu_fill_bf16}[kind]
    rc = fn(key, first, n, scale_const(std), out_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth GPU fill failed with hipError {rc}")


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Reinterpret bf16 storage bits as the float32 numbers they denote."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------------------
# Layer-level tensors.  kind(...) tells how a tensor is stored on the GPU side.

def token_kind(cfg: LayerConfig) -> str:
    return "f32" if cfg.dtype == "f32" else "bf16"


def router_kind(cfg: LayerConfig) -> str:
    return "f32" if cfg.dtype == "f32" else "bf16"


def expert_kind(cfg: LayerConfig) -> str:
    """Storage of the generated expert weights: bf16 values, or fp32 (f32 layers and fp8 master values)."""
    return "bf16" if cfg.dtype == "bf16" else "f32"


def _values(key: int, n: int, std: float, kind: str, first: int = 0) -> np.ndarray:
    v = host_fill(key, n, std, kind, first)
    return bf16_bits_as_f32(v) if kind == "bf16" else v


def tokens_key(cfg: LayerConfig, layer: int = 0) -> int:
    return tensor_key(SEED, cfg.wid, layer, TENSOR_X, 0)


def tokens(cfg: LayerConfig, layer: int = 0, rows: np.ndarray | None = None) -> np.ndarray:
    """Tokens x [T, H] (or only the given token rows) as float32 numbers."""
    key = tokens_key(cfg, layer)
    kind = token_kind(cfg)
    if rows is None:
        return _values(key, cfg.T * cfg.H, 1.0, kind).reshape(cfg.T, cfg.H)
    out = np.empty((len(rows), cfg.H), np.float32)
    for i, t in enumerate(rows):
        out[i] = _values(key, cfg.H, 1.0, kind, first=int(t) * cfg.H)
    return out


def router_key(cfg: LayerConfig, layer: int = 0) -> int:
    return tensor_key(SEED, cfg.wid, layer, TENSOR_ROUTER, 0)


def router_weight(cfg: LayerConfig, layer: int = 0) -> np.ndarray:
    """Router weight [E, H] as float32 numbers, ~N(0, 1/H)."""
    return _values(router_key(cfg, layer), cfg.E * cfg.H, 1.0 / math.sqrt(cfg.H),
                   router_kind(cfg)).reshape(cfg.E, cfg.H)


def router_bias(cfg: LayerConfig, layer: int = 0) -> np.ndarray | None:
    """Per-expert router-logit bias [E] float32, or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal":
        key = tensor_key(SEED, cfg.wid, layer, TENSOR_BIAS, 0)
        return host_fill(key, cfg.E, math.sqrt(0.5), "f32")
    if cfg.bias == "zipf":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg.wid, layer, 77])))
        rank = rng.permutation(cfg.E)           # popularity rank of each expert, 0 = most popular
        return (-1.1 * np.log(rank.astype(np.float64) + 1.0)).astype(np.float32)
    raise ValueError(cfg.bias)


def seq_lengths(cfg: LayerConfig) -> np.ndarray:
    """Sequence lengths of a multi-sequence batch (uniform integers in [seq_lo, seq_hi])."""
    if not cfg.n_seqs:
        return np.array([cfg.T])
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg.wid, 99])))
    return rng.integers(cfg.seq_lo, cfg.seq_hi + 1, size=cfg.n_seqs)


def expert_keys(cfg: LayerConfig, e: int, layer: int = 0) -> tuple[int, int, int]:
    """Keys of (Wg, Wu, Wd) of expert e; e == E is the shared expert."""
    return tuple(tensor_key(SEED, cfg.wid, layer, t, e) for t in (TENSOR_WG, TENSOR_WU, TENSOR_WD))


def expert_stds(cfg: LayerConfig) -> tuple[float, float, float]:
    return (1.0 / math.sqrt(cfg.H), 1.0 / math.sqrt(cfg.H), 1.0 / math.sqrt(cfg.I))


def expert_weights(cfg: LayerConfig, e: int, layer: int = 0):
    """(Wg [I,H], Wu [I,H], Wd [H,I]) of expert e as float32 numbers; e == E is the shared expert."""
    kg, ku, kd = expert_keys(cfg, e, layer)
    sg, su, sd = expert_stds(cfg)
    kind = expert_kind(cfg)
    wg = _values(kg, cfg.I * cfg.H, sg, kind).reshape(cfg.I, cfg.H)
    wu = _values(ku, cfg.I * cfg.H, su, kind).reshape(cfg.I, cfg.H)
    wd = _values(kd, cfg.H * cfg.I, sd, kind).reshape(cfg.H, cfg.I)
    return wg, wu, wd
