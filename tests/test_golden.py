"""The oracle against the stored fixtures in tests/golden (each file cites its source)."""
import os

import numpy as np

from oracle import codecs, moe
from oracle.prefetch import chunk_plan

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(HERE, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_e4m3_codes_from_the_format_definition():
    rows = lines("e4m3_codes.txt")
    dec = [(int(c, 16), float(v)) for kind, c, v in rows if kind == "decode"]
    enc = [(float(v), int(c, 16)) for kind, v, c in rows if kind == "encode"]
    assert dec and enc
    got = codecs.e4m3_decode(np.array([c for c, _ in dec], np.uint8))
    np.testing.assert_array_equal(got, np.array([v for _, v in dec]))
    codes = codecs.e4m3_encode(np.array([v for v, _ in enc]))
    np.testing.assert_array_equal(codes, np.array([c for _, c in enc], np.uint8))


def test_fp8_overlap_slice_plan():
    rows = {r[0]: r[1:] for r in lines("prefetch_plan_fp8_overlap.txt") if r[0] not in ("first", "last")}
    firsts = [tuple(map(int, r[1:])) for r in lines("prefetch_plan_fp8_overlap.txt") if r[0] == "first"]
    lasts = [tuple(map(int, r[1:])) for r in lines("prefetch_plan_fp8_overlap.txt") if r[0] == "last"]
    plan = chunk_plan([int(v) for v in rows["source_bytes"]], [int(v) for v in rows["dst_offsets"]],
                      int(rows["chunk_bytes"][0]))
    assert len(plan) == int(rows["n_slices"][0])
    assert [tuple(p) for p in plan[:len(firsts)]] == firsts
    assert [tuple(p) for p in plan[-len(lasts):]] == lasts


def _group(amax, value=None):
    """One 128-wide group: amax in column 0, `value` (if any) in column 1, zeros elsewhere."""
    g = np.zeros((1, 128), np.float32)
    g[0, 0] = amax
    if value is not None:
        g[0, 1] = value
    return g


def test_fp8_group_scales_and_codes():
    rows = lines("fp8_group_scales.txt")
    scales = [(float(a), int(b, 16)) for kind, a, b in (r for r in rows if r[0] == "scale")]
    codes = [(float(a), float(v), int(c, 16)) for kind, a, v, c in (r for r in rows if r[0] == "code")]
    assert scales and codes
    for amax, bits in scales:
        _, s = moe.quantize_groups(_group(amax))
        assert s.dtype == np.float32 and int(s.view(np.uint32)[0, 0]) == bits, (amax, hex(int(s.view(np.uint32)[0, 0])))
        blk = np.zeros((128, 128), np.float32)
        blk[5, 7] = amax
        _, sb = moe.quantize_blocks(blk)
        assert int(sb.view(np.uint32)[0, 0]) == bits, amax
    for amax, v, code in codes:
        q, _ = moe.quantize_groups(_group(amax, v))
        assert int(q[0, 1]) == code, (amax, v, hex(int(q[0, 1])))
        blk = np.zeros((128, 128), np.float32)
        blk[0, 0] = amax
        blk[100, 3] = v
        qb, _ = moe.quantize_blocks(blk)
        assert int(qb[100, 3]) == code, (amax, v)
