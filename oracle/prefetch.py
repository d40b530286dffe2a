"""Chunk plan of the layer-ahead expert prefetch (oracle; test infrastructure only).

While a rank runs layer l it pulls layer l+1's non-local experts into the other
half of a double buffer (DWDP paper summary, §2).  The pulls are cut into
fixed-size slices issued round-robin across the transfer queues, so that no
single large pull holds the copy engine (§4.3.2, time-division multiplexing).
Reading taken here: one queue per source region; slice c of every source is
issued before slice c+1 of any source; sources are visited in their given
order; the last slice of a source is whatever remains (possibly short).
"""
from __future__ import annotations

import numpy as np


def chunk_plan(sizes, dst_offsets, chunk: int):
    """List of (source, src_offset, dst_offset, length) in issue order."""
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    n_chunks = [-(-int(b) // chunk) for b in sizes]
    plan = []
    for c in range(max(n_chunks, default=0)):
        for s, b in enumerate(sizes):
            if c < n_chunks[s]:
                off = c * chunk
                plan.append((s, off, int(dst_offsets[s]) + off, min(chunk, int(b) - off)))
    return plan


def apply_plan(dst: np.ndarray, sources, dst_offsets, chunk: int) -> np.ndarray:
    """The destination bytes after running the plan (dst and sources are uint8 arrays)."""
    out = np.array(dst, dtype=np.uint8, copy=True)
    for s, so, do, n in chunk_plan([len(x) for x in sources], dst_offsets, chunk):
        out[do:do + n] = sources[s][so:so + n]
    return out
