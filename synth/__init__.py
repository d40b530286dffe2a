"""Seeded synthetic inputs for the one-rank DWDP MoE block.

Test and benchmark infrastructure, shared by the GPU path and the CPU oracle.
It produces inputs (tokens, router weights, router bias, expert weights, the
expert placement split and sequence lengths) and holds none of the MoE
layer's arithmetic: no routing, permutation, GEMM, activation, quantisation
or combine.

Every tensor is identified by a tuple (seed, workload id, layer, tensor id,
expert) hashed to a 64-bit key; element i of the tensor is a pure function of
(key, i), so any slice of any tensor can be produced on either side without
producing the rest.  The element generator is written twice, in C for the host
(`synth_host.c`) and in HIP for the GPU (`synth_gpu.hip`); the two must agree
bit for bit.
"""
from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    TENSOR_X, TENSOR_ROUTER, TENSOR_BIAS, TENSOR_WG, TENSOR_WU, TENSOR_WD,
    tensor_key, scale_const, host_fill, host_gather, gpu_fill,
    tokens, router_weight, router_bias, expert_weights, seq_lengths,
)
