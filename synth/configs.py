"""The five synthetic MoE-layer workloads.

Shapes follow a DeepSeek-R1-sized MoE layer (hidden 7168, expert intermediate
2048, 256 routed experts, top-8, one always-on shared expert) plus a tiny fp32
layer that an fp64 oracle evaluates in well under a second.  The pages measure
DeepSeek-R1 serving with 8K input / 1K output sequences, input lengths between
0.8x8K and 8K per rank, and context lengths up to 32K (DWDP paper summary,
§1 Fig. 1 and §5.2 Table 3); these synthetic layers stand in for that
workload.  No trained weights or datasets are involved.

Placement: DWDP with a group of four ranks keeps a quarter of each layer's
routed experts resident and pulls the other three quarters from three peers
(paper summary §2 and §4.1.1 Table 1, DWDP4).  Here experts [0, n_local) and
the shared expert are resident; the rest sit in `n_sources` stand-in source
regions of equal size and are copied into a prefetch slot set.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math


@dataclass(frozen=True)
class LayerConfig:
    name: str
    wid: int            # workload id, part of every tensor's seed tuple
    T: int              # tokens in the batch (sum of seq_lens when given)
    H: int              # hidden size
    I: int              # expert intermediate size
    E: int              # routed experts
    k: int              # experts per token
    shared: int         # 1 = one always-on shared expert of the same shape
    dtype: str          # "f32" | "bf16" | "fp8"
    bias: str           # "none" | "normal" (N(0, 0.5) per expert) | "zipf" (s = 1.1)
    n_local: int        # routed experts [0, n_local) are resident
    n_sources: int      # stand-in source regions holding experts [n_local, E)
    chunk_bytes: int = 4 << 20
    n_seqs: int = 0     # >0: T is the sum of n_seqs lengths drawn from [lo, hi]
    seq_lo: int = 0
    seq_hi: int = 0
    note: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        """Routed rows, T*k."""
        return self.T * self.k

    @property
    def rows(self) -> int:
        """Rows of the permuted activation matrix: routed rows plus T shared rows."""
        return self.T * self.k + self.shared * self.T

    @property
    def groups(self) -> int:
        return self.E + self.shared

    @property
    def n_prefetch(self) -> int:
        return self.E - self.n_local

    def flops_ffn(self, rows: int | None = None) -> int:
        """Algorithmic FLOPs of the expert FFNs: 6*H*I per (token, expert) row."""
        r = self.rows if rows is None else rows
        return 6 * self.H * self.I * r

    def flops_router(self) -> int:
        return 2 * self.T * self.H * self.E

    def weight_bytes_per_expert(self) -> int:
        """Bytes of one expert's weight record (W13, W2 and, for fp8, block scales)."""
        n = 3 * self.H * self.I
        if self.dtype == "f32":
            return 4 * n
        if self.dtype == "bf16":
            return 2 * n
        nb13 = (2 * self.I // 128) * (self.H // 128)
        nb2 = (self.H // 128) * (self.I // 128)
        return n + 4 * (nb13 + nb2)


_SEQ_LO = math.ceil(0.8 * 8192)   # 6554

CONFIGS = {
    c.name: c
    for c in [
        LayerConfig("tiny_f32", 0, T=64, H=256, I=128, E=8, k=2, shared=0, dtype="f32", bias="none",
                    n_local=4, n_sources=1,
                    note="tiny fp32 layer; experts 0-3 resident, 4-7 in a separate prefetch buffer"),
        LayerConfig("prefill8k_bf16", 1, T=8192, H=7168, I=2048, E=256, k=8, shared=1, dtype="bf16",
                    bias="normal", n_local=64, n_sources=3,
                    note="8K-token bf16 prefill chunk, per-expert N(0,0.5) router-logit bias"),
        LayerConfig("imbalanced_bf16", 2, T=0, H=7168, I=2048, E=256, k=8, shared=1, dtype="bf16",
                    bias="zipf", n_local=64, n_sources=3, n_seqs=4, seq_lo=_SEQ_LO, seq_hi=8192,
                    note="4 sequences of U{6554..8192} tokens, Zipf(1.1) expert popularity bias"),
        LayerConfig("decode64_bf16", 3, T=64, H=7168, I=2048, E=256, k=8, shared=1, dtype="bf16",
                    bias="none", n_local=64, n_sources=3,
                    note="64-token decode step, weight streaming"),
        LayerConfig("prefill16k_fp8", 4, T=16384, H=7168, I=2048, E=256, k=8, shared=1, dtype="fp8",
                    bias="none", n_local=64, n_sources=3,
                    note="16K-token fp8 prefill, 128x128 weight blocks, 1x128 activation groups, "
                         "next layer's 192 experts prefetched concurrently"),
    ]
}


def get_config(name: str) -> LayerConfig:
    """Return the named workload; the imbalanced batch gets its T from its drawn lengths."""
    cfg = CONFIGS[name]
    if cfg.n_seqs and cfg.T == 0:
        from .gen import seq_lengths
        from dataclasses import replace
        cfg = replace(cfg, T=int(sum(seq_lengths(cfg))))
    return cfg


def shrink(cfg: LayerConfig, **kw) -> LayerConfig:
    """A copy of `cfg` with some fields replaced (small parity cases of a large workload)."""
    from dataclasses import replace
    return replace(cfg, **kw)
