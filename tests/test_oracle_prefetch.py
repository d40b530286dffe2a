"""Pins of the oracle's round-robin chunk plan: coverage, order and the short last slice."""
import numpy as np
import pytest

from oracle.prefetch import apply_plan, chunk_plan


def test_plan_hand_example():
    # sources of 10, 4 and 0 bytes, chunk 4: slice 0 of each, then slice 1 of the first, ...
    plan = chunk_plan([10, 4, 0], [0, 100, 200], 4)
    assert plan == [(0, 0, 0, 4), (1, 0, 100, 4), (0, 4, 4, 4), (0, 8, 8, 2)]


def test_plan_round_robin_order_and_partial_last_chunk():
    sizes = [4 * 1024 * 1024 * 3 + 688128] * 3
    plan = chunk_plan(sizes, [0, sizes[0], 2 * sizes[0]], 4 * 1024 * 1024)
    assert len(plan) == 12
    assert [p[0] for p in plan] == [0, 1, 2] * 4
    assert all(p[3] == 4 * 1024 * 1024 for p in plan[:9]) and all(p[3] == 688128 for p in plan[9:])


@pytest.mark.parametrize("seed", range(20))
def test_plan_covers_every_byte_exactly_once(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 6))
    sizes = [int(s) for s in rng.integers(0, 3000, size=n)]
    chunk = int(rng.integers(1, 700))
    gaps = rng.integers(0, 50, size=n)
    dst_off = np.cumsum(np.concatenate([[0], np.array(sizes[:-1]) + gaps[:-1]])).astype(int)
    hits = np.zeros(int(dst_off[-1]) + sizes[-1] + 1, int)
    for s, so, do, ln in chunk_plan(sizes, dst_off, chunk):
        assert 0 < ln <= chunk and so % chunk == 0
        assert do - dst_off[s] == so
        hits[do:do + ln] += 1
    for s in range(n):
        assert np.all(hits[dst_off[s]:dst_off[s] + sizes[s]] == 1)
    assert hits.sum() == sum(sizes)
    srcs = [rng.integers(0, 256, size=b, dtype=np.uint8) for b in sizes]
    dst = np.zeros(len(hits), np.uint8)
    out = apply_plan(dst, srcs, dst_off, chunk)
    for s in range(n):
        np.testing.assert_array_equal(out[dst_off[s]:dst_off[s] + sizes[s]], srcs[s])
