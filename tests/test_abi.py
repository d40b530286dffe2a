"""The C ABI without a GPU: the library loads, exports every declared symbol,
rejects bad arguments before launching anything, and its host-only logic
(slice plan, record layout, pointer table, workspace sizes) is right."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle.prefetch import chunk_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dwdp.h")

lib_mod = pytest.importorskip("split_weight_expert_amd._lib")


@pytest.fixture(scope="module")
def lib():
    return lib_mod.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dwdp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(lib_mod.SIGNATURES), "binding signatures and header disagree"


def test_version_and_empty_error(lib):
    assert b"gfx950" in lib.dwdp_version()
    assert lib.dwdp_last_error() == b""


FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x10004)


def expect(code, rc, lib, needle):
    assert rc == code, (rc, lib.dwdp_last_error())
    assert needle in lib.dwdp_last_error().decode()


def test_route_topk_rejects_bad_arguments(lib):
    f = lib.dwdp_route_topk
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    expect(E_, f(FAKE, FAKE, 7, None, 4, 256, 8, 2, FAKE, FAKE, FAKE, None), lib, "in_dtype")
    expect(E_, f(FAKE, FAKE, 0, None, 4, 256, 8, 9, FAKE, FAKE, FAKE, None), lib, "k must")
    expect(E_, f(FAKE, FAKE, 0, None, 4, 256, 8, 0, FAKE, FAKE, FAKE, None), lib, "k must")
    expect(E_, f(FAKE, FAKE, 1, None, 4, 100, 8, 2, FAKE, FAKE, FAKE, None), lib, "H % 64")
    expect(E_, f(None, FAKE, 0, None, 4, 256, 8, 2, FAKE, FAKE, FAKE, None), lib, "null")
    expect(E_, f(ODD, FAKE, 0, None, 4, 256, 8, 2, FAKE, FAKE, FAKE, None), lib, "aligned")
    assert f(None, None, 0, None, 0, 256, 8, 2, None, None, None, None) == 0      # T = 0 is a no-op


def test_permute_rejects_bad_arguments(lib):
    f = lib.dwdp_permute
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    base = dict(idx=FAKE, T=4, k=2, E=8, S=0, x=FAKE, xd=1, ad=1, H=256, xp=FAKE, xs=None, off=FAKE, ps=FAKE,
                ip=FAKE, ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = {**base, **kw}
        return f(a["idx"], a["T"], a["k"], a["E"], a["S"], a["x"], a["xd"], a["ad"], a["H"], a["xp"], a["xs"],
                 a["off"], a["ps"], a["ip"], a["ws"], a["wsb"], None)
    expect(E_, call(S=2), lib, "shared")
    expect(E_, call(ad=2, xd=0), lib, "act_dtype")
    expect(E_, call(ad=2, xs=None), lib, "x_perm_scale")
    expect(E_, call(ad=2, H=200, xs=FAKE), lib, "H % 128")
    expect(E_, call(ps=None), lib, "null")
    expect(E_, call(xp=FAKE, x=None), lib, "x is NULL")
    expect(lib_mod.DWDP_ERR_WORKSPACE, call(wsb=16), lib, "workspace")


def test_grouped_ffn_rejects_bad_arguments(lib):
    f = lib.dwdp_moe_grouped_ffn
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    expect(E_, f(FAKE, 9, FAKE, FAKE, None, 128, 7168, 2048, 5, FAKE, FAKE, 1 << 30, None), lib, "w_dtype")
    expect(E_, f(FAKE, 9, FAKE, FAKE, None, 128, 7040, 2048, 1, FAKE, FAKE, 1 << 30, None), lib, "H % 256")
    expect(E_, f(FAKE, 9, FAKE, FAKE, None, 128, 7168, 2048, 2, FAKE, FAKE, 1 << 30, None), lib, "activation scales")
    expect(E_, f(FAKE, 9, FAKE, ODD, None, 128, 7168, 2048, 1, FAKE, FAKE, 1 << 30, None), lib, "aligned")
    expect(lib_mod.DWDP_ERR_WORKSPACE, f(FAKE, 9, FAKE, FAKE, None, 128, 7168, 2048, 1, FAKE, FAKE, 64, None),
           lib, "workspace")
    assert f(None, 9, None, None, None, 0, 7168, 2048, 1, None, None, 0, None) == 0   # rows = 0


def test_token_rows_ffn_and_token_quantiser_reject_bad_arguments(lib):
    f = lib.dwdp_moe_grouped_ffn_tokens
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    # stage, table, n_groups, offsets, perm_src, x, x_scale, T, rows, H, I, w_dtype, y_perm, ws, ws_bytes, stream
    expect(E_, f(0, FAKE, 9, FAKE, None, FAKE, None, 16, 128, 7168, 2048, 1, FAKE, FAKE, 1 << 30, None), lib,
           "perm_src")
    expect(E_, f(0, FAKE, 9, FAKE, FAKE, FAKE, None, 0, 128, 7168, 2048, 1, FAKE, FAKE, 1 << 30, None), lib, "T must")
    expect(E_, f(3, FAKE, 9, FAKE, FAKE, FAKE, None, 16, 128, 7168, 2048, 1, FAKE, FAKE, 1 << 30, None), lib, "stage")
    expect(E_, f(0, FAKE, 9, FAKE, FAKE, FAKE, None, 16, 128, 7168, 2048, 2, FAKE, FAKE, 1 << 30, None), lib,
           "activation scales")
    expect(lib_mod.DWDP_ERR_WORKSPACE, f(0, FAKE, 9, FAKE, FAKE, FAKE, None, 16, 128, 7168, 2048, 1, FAKE, FAKE, 64,
                                         None), lib, "workspace")
    assert f(0, None, 9, None, None, None, None, 0, 0, 7168, 2048, 1, None, None, 0, None) == 0   # rows = 0
    q = lib.dwdp_quantize_tokens_fp8
    expect(E_, q(FAKE, 4, 100, FAKE, FAKE, None), lib, "multiple of 128")
    expect(E_, q(ODD, 4, 128, FAKE, FAKE, None), lib, "aligned")
    expect(E_, q(FAKE, 4, 128, FAKE, None, None), lib, "null")
    assert q(None, 0, 128, None, None, None) == 0


def test_combine_and_prefetch_reject_bad_arguments(lib):
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    expect(E_, lib.dwdp_combine(FAKE, FAKE, FAKE, 4, 2, 0, 100, 1, FAKE, None), lib, "multiple of 8")
    expect(E_, lib.dwdp_combine(FAKE, FAKE, FAKE, 4, 2, 3, 128, 1, FAKE, None), lib, "shared")
    srcs = (lib_mod.CopySrc * 2)()
    srcs[0].src, srcs[0].dst_offset, srcs[0].bytes = 0x10000, 0, 100
    srcs[1].src, srcs[1].dst_offset, srcs[1].bytes = 0x20000, 50, 100
    expect(E_, lib.dwdp_prefetch_chunks(FAKE, srcs, 2, 16, 0, 0, None, None, None), lib, "overlap")
    srcs[1].dst_offset = 100
    expect(E_, lib.dwdp_prefetch_chunks(FAKE, srcs, 2, 0, 0, 0, None, None, None), lib, "chunk_bytes")
    expect(E_, lib.dwdp_prefetch_chunks(FAKE, srcs, 2, 16, 9, 0, None, None, None), lib, "engine")
    expect(E_, lib.dwdp_prefetch_chunks(FAKE, srcs, 0, 16, 0, 0, None, None, None), lib, "n_src")


@pytest.mark.parametrize("seed", range(10))
def test_prefetch_plan_matches_oracle(seed):
    from split_weight_expert_amd import api
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    sizes = [int(s) for s in rng.integers(0, 5000, size=n)]
    chunk = int(rng.integers(1, 900))
    offs = np.cumsum([0] + [s + 7 for s in sizes[:-1]]).tolist()
    srcs = [(0x1000 * (i + 1), offs[i], sizes[i]) for i in range(n)]
    got = api.prefetch_plan(srcs, chunk)
    assert got == chunk_plan(sizes, offs, chunk)


def test_prefetch_plan_for_the_fp8_overlap_workload():
    from split_weight_expert_amd import api
    rec = api.expert_record_bytes(7168, 2048, 2)
    assert rec == 44_050_944
    per = 64 * rec
    plan = api.prefetch_plan([(0x1000, 0, per), (0x2000, per, per), (0x3000, 2 * per, per)], 4 << 20)
    assert len(plan) == 3 * 673 and plan[-1][3] == 688_128
    assert [p[0] for p in plan[:6]] == [0, 1, 2, 0, 1, 2]


def test_record_layout_and_pointer_table():
    from split_weight_expert_amd import api
    assert api.expert_record_bytes(7168, 2048, 1) == 88_080_384
    w2, s13, s2 = api.expert_record_offsets(7168, 2048, 2)
    assert w2 == 2 * 2048 * 7168 and s13 == w2 + 7168 * 2048 and s2 == s13 + 1792 * 4
    rec = api.expert_record_bytes(256, 128, 0)
    t = api.fill_expert_table([0x100000, 0x900000], [0, 1, 1, 0], [0, 0, 3, 2], 256, 128, 0)
    assert t[0].w13 == 0x100000 and t[1].w13 == 0x900000 and t[2].w13 == 0x900000 + 3 * rec
    assert t[3].w2 == 0x100000 + 2 * rec + 2 * 128 * 256 * 4
    assert t[0].s13 is None and t[0].s2 is None
    with pytest.raises(lib_mod.DwdpError):
        api.fill_expert_table([0x100000], [1], [0], 256, 128, 0)


def test_workspace_sizes_grow_with_rows():
    from split_weight_expert_amd import api
    a = api.workspace_bytes(api.OP_GROUPED_FFN, 8192, 8, 256, 7168, 2048, 1, 1)
    b = api.workspace_bytes(api.OP_GROUPED_FFN, 64, 8, 256, 7168, 2048, 1, 1)
    assert a >= 73728 * 2048 * 2 and b >= 576 * 2048 * 2 and a > b
    assert api.workspace_bytes(api.OP_PERMUTE, 8192, 8, 256, 7168, 2048, 1, 1) > 0


def test_grouped_ffn_rejects_shapes_outside_the_documented_limits(lib):
    """The header's limits are what the library enforces: f32 needs H % 64 and I % 32, bf16/fp8 H % 256 and
    I % 128, fp8 also H, I <= 8192."""
    f = lib.dwdp_moe_grouped_ffn
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    ws = 1 << 40
    for H, I, dt in ((96, 128, 0), (256, 48, 0), (7040, 2048, 1), (7168, 2000, 1), (8448, 2048, 2)):
        expect(E_, f(FAKE, 9, FAKE, FAKE, FAKE, 128, H, I, dt, FAKE, FAKE, ws, None), lib, "H")
    for H, I, dt in ((64, 32, 0), (256, 128, 1), (8192, 8192, 2)):   # accepted shapes fail later (on `rows`)
        rc = f(FAKE, 9, FAKE, FAKE, FAKE, -1, H, I, dt, FAKE, FAKE, ws, None)
        assert rc == E_ and "rows" in lib.dwdp_last_error().decode(), (H, I, dt)


def test_store_rejects_placements_outside_its_buffers():
    """ExpertStore.table checks every (buffer, slot) against the store before filling the pointer table (the
    C ABI cannot: it does not know the buffers' sizes)."""
    import torch

    from split_weight_expert_amd import ExpertStore
    st = ExpertStore(256, 128, lib_mod.F32, [2, 3], device="cpu")
    good = [(0, 0), (0, 1), (1, 2)]
    t = st.table(good, "cpu")
    assert t.numel() == 32 * len(good)
    for bad in ([(0, 2)], [(1, 3)], [(2, 0)], [(0, -1)], [(-1, 0)]):
        with pytest.raises(ValueError):
            st.table(good + bad, "cpu")
    del torch


def test_launch_sizes_beyond_one_dispatch_are_rejected(lib):
    """A dispatch holds fewer than 2^32 work-items.  The per-row and per-token kernels walk any count with a
    bounded grid; the tiled GEMMs reject a problem whose tile grid would not fit, before anything is
    launched (the pointers here are never dereferenced)."""
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    # router: 2^30 tokens of 1024 experts is 2^28 tiles of 64 x 64
    expect(E_, lib.dwdp_route_topk(FAKE, FAKE, 1, None, 1 << 30, 64, 1024, 8, FAKE, FAKE, FAKE, None), lib,
           "too large")
    # grouped FFN: 2^31 - 1 rows in one group is 2^23 tiles of 256 rows, times 512 work-items
    rows = (1 << 31) - 1
    expect(E_, lib.dwdp_moe_grouped_ffn(FAKE, 1, FAKE, FAKE, None, rows, 256, 128, 1, FAKE, FAKE, 1 << 62, None), lib,
           "too large")


def test_diagnostics_reject_bad_arguments_and_the_default_build_has_no_tile_trace(lib):
    f = lib.dwdp_diag_operand_stream
    E_ = lib_mod.DWDP_ERR_INVALID_ARG
    MiB = 1 << 20
    expect(E_, f(None, MiB, 0, 1, 1, 3, 0, None), lib, "NULL")
    expect(E_, f(ODD, MiB, 0, 1, 1, 3, 0, None), lib, "aligned")
    expect(E_, f(FAKE, MiB + 16, 0, 1, 1, 3, 0, None), lib, "32768")
    expect(E_, f(FAKE, 0, 0, 1, 1, 3, 0, None), lib, "32768")
    expect(E_, f(FAKE, MiB, 8, 1, 1, 3, 0, None), lib, "stride")
    expect(E_, f(FAKE, MiB, 0, 0, 1, 3, 0, None), lib, "iters")
    expect(E_, f(FAKE, MiB, 0, 1, 0, 3, 0, None), lib, "grid")
    expect(E_, f(FAKE, MiB, 0, 1, 65537, 3, 0, None), lib, "grid")
    expect(E_, f(FAKE, MiB, 0, 1, 1, 0, 0, None), lib, "in_flight")
    expect(E_, f(FAKE, MiB, 0, 1, 1, 6, 0, None), lib, "in_flight")
    expect(E_, f(FAKE, MiB, 0, 1, 1, 3, 1, None), lib, "cpol")
    g = lib.dwdp_diag_lds_read
    expect(E_, g(0, 8, 1, FAKE, FAKE, None), lib, "grid")
    expect(E_, g(1, 6, 1, FAKE, FAKE, None), lib, "waves")
    expect(E_, g(1, 8, 0, FAKE, FAKE, None), lib, "iters")
    expect(E_, g(1, 8, 1, None, FAKE, None), lib, "null")
    expect(E_, g(1, 8, 1, FAKE, ODD, None), lib, "aligned")
    assert ctypes.sizeof(lib_mod.TileRecord) == 48
    n = ctypes.c_size_t(7)
    buf = (lib_mod.TileRecord * 4)()
    expect(E_, lib.dwdp_diag_tile_trace_read(None, 4, ctypes.byref(n)), lib, "null")
    if b"tile-trace=1" not in lib.dwdp_version():
        U = lib_mod.DWDP_ERR_UNSUPPORTED
        expect(U, lib.dwdp_diag_tile_trace_clear(None), lib, "DWDP_TILE_TRACE")
        expect(U, lib.dwdp_diag_tile_trace_read(buf, 4, ctypes.byref(n)), lib, "DWDP_TILE_TRACE")
        assert n.value == 7
