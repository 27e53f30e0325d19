"""CPU checks of the C ABI: the library loads, exports every declared symbol, the
planners match the oracle's planner, and every invalid-argument path returns its status
before touching the GPU (these calls pass fake, aligned device addresses, which the
library never dereferences on the host)."""

import ctypes
import os
import re

import pytest

import oracle
import mla_split_kv_02_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mla.LIB_PATH), reason="library not built")

F = 0x10000000  # fake 256-aligned device address (never dereferenced by failing calls)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = mla.lib()
    decl = declared_functions()
    assert decl == sorted(mla.EXPORTED_SYMBOLS)
    for name in decl:
        assert hasattr(L, name), name


def test_ceiling_library_exports_its_header():
    from mla_split_kv_02_amd import ceiling
    if not os.path.exists(ceiling.CEILING_LIB_PATH):
        pytest.skip("measurement library not built")
    text = open(os.path.join(ROOT, "include", "mla_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decl = sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))
    assert decl == sorted(ceiling.EXPORTED_SYMBOLS)
    L = ceiling.lib()
    for name in decl:
        assert hasattr(L, name), name
    assert L.mla_ceiling_mfma_flops(0) == 32768.0 and L.mla_ceiling_mfma_flops(1) == 131072.0
    assert L.mla_ceiling_mfma_flops(2) == 32768.0 and L.mla_ceiling_mfma_flops(3) == 0.0
    # invalid arguments are refused before any launch
    assert L.mla_ceiling_stream_read(None, 16, None, 1, None) == -1
    assert L.mla_ceiling_mfma(7, 1, ctypes.c_void_p(F), 1, None) == -1
    assert L.mla_ceiling_mfma(3, 1, ctypes.c_void_p(F), 1, None) == -1


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert mla.status_string(s).startswith("MLA_")
    assert mla.status_string(7) == "unknown mla_status"


def test_plan_contig_matches_oracle():
    for cus in (1, 80, 256, 304):
        for B in (1, 2, 3, 4, 32, 64, 255, 256, 1000):
            for S in (1, 100, 128, 129, 256, 4096, 8192, 65537):
                assert mla.plan_contig(cus, B, S) == oracle.plan_contig(cus, B, S), (cus, B, S)


def test_plan_paged_and_workspace():
    assert mla.plan_paged(256, 64, 1, 128) == 256
    assert mla.plan_paged(256, 128, 2, 128) == 128
    assert mla.plan_paged(256, 4, 1, 16) == 256
    assert mla.plan_paged(1, 4, 8, 128) == 1
    ws = mla.paged_workspace_bytes(64, 1, 128, 256)
    per_split = oracle.workspace_floats_per_split(1, 128) * 4
    assert ws >= (256 + 63) * per_split
    assert ws < (256 + 63) * per_split + 4096
    assert mla.paged_workspace_bytes(0, 1, 128, 256) == 0
    assert mla.paged_workspace_bytes(4, 9, 128, 256) == 0
    assert mla.paged_workspace_bytes(4, 1, 24, 256) == 0


def _paged(**kw):
    a = dict(q=F, qpe=F, cache=F, fmt=1, kv_scale=1.0, num_pages=10, page_size=64, stride=64 * 576, bt=F, mb=4,
             sl=F, B=2, q_len=1, H=128, sm=0.07, ns=8, ws=F, ws_bytes=1 << 30, o=F, lse=F)
    a.update(kw)
    vp = ctypes.c_void_p
    return mla.lib().mla_paged_decode(vp(a["q"]), vp(a["qpe"]), vp(a["cache"]), a["fmt"], a["kv_scale"],
                                      a["num_pages"], a["page_size"], a["stride"], vp(a["bt"]), a["mb"],
                                      vp(a["sl"]), a["B"], a["q_len"], a["H"], a["sm"], a["ns"], vp(a["ws"]),
                                      a["ws_bytes"], vp(a["o"]), vp(a["lse"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), mla.MLA_ERR_INVALID_ARG),
    (dict(cache=0), mla.MLA_ERR_INVALID_ARG),
    (dict(bt=0), mla.MLA_ERR_INVALID_ARG),
    (dict(sl=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ws=0), mla.MLA_ERR_INVALID_ARG),
    (dict(o=0), mla.MLA_ERR_INVALID_ARG),
    (dict(q=F + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(ws=F + 16), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=4), mla.MLA_ERR_UNSUPPORTED),
    (dict(fmt=-1), mla.MLA_ERR_UNSUPPORTED),
    (dict(page_size=16), mla.MLA_ERR_UNSUPPORTED),
    (dict(page_size=128), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_len=0), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_len=9), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=24), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=144), mla.MLA_ERR_UNSUPPORTED),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(B=4097), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=65537), mla.MLA_ERR_INVALID_ARG),
    (dict(stride=64 * 576 - 16), mla.MLA_ERR_INVALID_ARG),
    (dict(stride=64 * 576 + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=0, stride=64 * 576), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=2, stride=64 * 324 - 16), mla.MLA_ERR_INVALID_ARG),
    (dict(num_pages=0), mla.MLA_ERR_INVALID_ARG),
    (dict(mb=0), mla.MLA_ERR_INVALID_ARG),
    (dict(B=4096, mb=1 << 14), mla.MLA_ERR_INVALID_ARG),
    (dict(kv_scale=0.0), mla.MLA_ERR_INVALID_ARG),
    (dict(kv_scale=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=3, kv_scale=0.0), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=3, stride=64 * 576 - 16), mla.MLA_ERR_INVALID_ARG),
    (dict(sm=float("inf")), mla.MLA_ERR_INVALID_ARG),
    (dict(sm=-0.125), mla.MLA_ERR_INVALID_ARG),
    (dict(ws_bytes=1000), mla.MLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_paged_decode_rejects(kw, status):
    assert _paged(**kw) == status


def test_paged_workspace_boundary():
    need = mla.paged_workspace_bytes(2, 1, 128, 8)
    assert _paged(ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL


def _contig(**kw):
    a = dict(q=F, qpe=F, kv=F, kpe=F, B=2, H=16, S=256, sm=0.07, L=128, op=F, lp=F)
    a.update(kw)
    vp = ctypes.c_void_p
    return mla.lib().mla_decode_splitkv(vp(a["q"]), vp(a["qpe"]), vp(a["kv"]), vp(a["kpe"]), a["B"], a["H"],
                                        a["S"], a["sm"], a["L"], vp(a["op"]), vp(a["lp"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), mla.MLA_ERR_INVALID_ARG),
    (dict(kpe=0), mla.MLA_ERR_INVALID_ARG),
    (dict(op=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lp=0), mla.MLA_ERR_INVALID_ARG),
    (dict(kv=F + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(L=100), mla.MLA_ERR_INVALID_ARG),
    (dict(L=64), mla.MLA_ERR_INVALID_ARG),
    (dict(L=384), mla.MLA_ERR_INVALID_ARG),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(S=0), mla.MLA_ERR_INVALID_ARG),
    (dict(H=8), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=136), mla.MLA_ERR_UNSUPPORTED),
    (dict(sm=float("nan")), mla.MLA_ERR_INVALID_ARG),
    (dict(sm=-1.0), mla.MLA_ERR_INVALID_ARG),
    (dict(B=65536), mla.MLA_ERR_INVALID_ARG),
    (dict(S=65536 * 128), mla.MLA_ERR_INVALID_ARG),        # 65536 splits
    (dict(B=32768, S=32769 * 128), mla.MLA_ERR_INVALID_ARG),  # NS * B > 2^30 workgroups
])
def test_decode_splitkv_rejects(kw, status):
    assert _contig(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(op=0), mla.MLA_ERR_INVALID_ARG),
    (dict(o=0), mla.MLA_ERR_INVALID_ARG),
    (dict(rows=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=65537), mla.MLA_ERR_INVALID_ARG),
    (dict(o=F + 4), mla.MLA_ERR_INVALID_ARG),
])
def test_combine_rejects(kw, status):
    a = dict(op=F, lp=F, rows=4, ns=2, o=F, lse=F)
    a.update(kw)
    vp = ctypes.c_void_p
    assert mla.lib().mla_splitkv_combine(vp(a["op"]), vp(a["lp"]), a["rows"], a["ns"], vp(a["o"]), vp(a["lse"]),
                                         None) == status


def test_planner_null_outputs():
    L = mla.lib()
    assert L.mla_plan_contig(256, 1, 256, None, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_plan_paged(256, 1, 1, 16, None) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_device_num_cus(0, None) == mla.MLA_ERR_INVALID_ARG


def test_paged_partials_and_combine_reject():
    L = mla.lib()
    vp = ctypes.c_void_p
    ws = mla.paged_workspace_bytes(2, 1, 128, 8)
    ok = (vp(F), vp(F), vp(F), 1, 1.0, 10, 64, 64 * 576, vp(F), 4, vp(F), 2, 1, 128, 0.07, 8, vp(F), ws, None)
    bad_fmt = ok[:3] + (5,) + ok[4:]
    assert L.mla_paged_decode_partials(*bad_fmt) == mla.MLA_ERR_UNSUPPORTED
    small_ws = ok[:17] + (ws - 1, None)
    assert L.mla_paged_decode_partials(*small_ws) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    null_q = (None,) + ok[1:]
    assert L.mla_paged_decode_partials(*null_q) == mla.MLA_ERR_INVALID_ARG
    c_ok = [vp(F), ws, vp(F), 2, 1, 128, 8, 4, 64, vp(F), vp(F), None]
    for i, v, st in ((0, None, mla.MLA_ERR_INVALID_ARG), (1, ws - 1, mla.MLA_ERR_WORKSPACE_TOO_SMALL),
                     (2, None, mla.MLA_ERR_INVALID_ARG), (5, 40, mla.MLA_ERR_UNSUPPORTED),
                     (8, 48, mla.MLA_ERR_UNSUPPORTED), (7, 0, mla.MLA_ERR_INVALID_ARG),
                     (9, None, mla.MLA_ERR_INVALID_ARG), (9, vp(F + 2), mla.MLA_ERR_INVALID_ARG)):
        args = list(c_ok)
        args[i] = v
        assert L.mla_paged_combine(*args) == st, (i, v)


def _append(**kw):
    a = dict(lat=F, rope=F, slots=F, T=4, cache=F, fmt=1, kv_scale=0.5, num_pages=10, page_size=64,
             stride=64 * 576)
    a.update(kw)
    vp = ctypes.c_void_p
    return mla.lib().mla_kv_append(vp(a["lat"]), vp(a["rope"]), vp(a["slots"]), a["T"], vp(a["cache"]), a["fmt"],
                                   a["kv_scale"], a["num_pages"], a["page_size"], a["stride"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(lat=0), mla.MLA_ERR_INVALID_ARG),
    (dict(rope=0), mla.MLA_ERR_INVALID_ARG),
    (dict(slots=0), mla.MLA_ERR_INVALID_ARG),
    (dict(cache=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lat=F + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(slots=F + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(cache=F + 8), mla.MLA_ERR_INVALID_ARG),
    (dict(T=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=4), mla.MLA_ERR_UNSUPPORTED),
    (dict(fmt=-1), mla.MLA_ERR_UNSUPPORTED),
    (dict(page_size=16), mla.MLA_ERR_UNSUPPORTED),
    (dict(num_pages=0), mla.MLA_ERR_INVALID_ARG),
    (dict(num_pages=1 << 25), mla.MLA_ERR_INVALID_ARG),
    (dict(stride=64 * 576 - 16), mla.MLA_ERR_INVALID_ARG),
    (dict(stride=64 * 576 + 4), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=0, stride=64 * 576), mla.MLA_ERR_INVALID_ARG),
    (dict(kv_scale=0.0), mla.MLA_ERR_INVALID_ARG),
    (dict(kv_scale=float("inf")), mla.MLA_ERR_INVALID_ARG),
])
def test_kv_append_rejects(kw, status):
    assert _append(**kw) == status


def test_kv_append_no_tokens_enqueues_nothing():
    # T = 0 is accepted before any pointer is looked at; nothing is launched
    assert _append(T=0, lat=0, rope=0, slots=0, cache=0) == mla.MLA_OK
    # kv_scale only matters for FP8
    assert _append(T=0, fmt=2, stride=64 * 324, kv_scale=0.0) == mla.MLA_OK


def _ext(**kw):
    a = dict(q=F, qpe=F, cache=F, fmt=1, kv_scale=1.0, num_pages=10, page_size=64, stride=64 * 576, bt=F, mb=4,
             sl=F, B=2, q_len=1, H=128, sm=0.07, win=0, sinks=0, ns=8, ws=F, ws_bytes=1 << 30, o=F, lse=F)
    a.update(kw)
    vp = ctypes.c_void_p
    return mla.lib().mla_paged_decode_ext(vp(a["q"]), vp(a["qpe"]), vp(a["cache"]), a["fmt"], a["kv_scale"],
                                          a["num_pages"], a["page_size"], a["stride"], vp(a["bt"]), a["mb"],
                                          vp(a["sl"]), a["B"], a["q_len"], a["H"], a["sm"], a["win"],
                                          vp(a["sinks"]), a["ns"], vp(a["ws"]), a["ws_bytes"], vp(a["o"]),
                                          vp(a["lse"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(win=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(sinks=F + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(q=0), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=4), mla.MLA_ERR_UNSUPPORTED),
    (dict(ws_bytes=1000), mla.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(o=F + 4), mla.MLA_ERR_INVALID_ARG),
])
def test_paged_decode_ext_rejects(kw, status):
    assert _ext(**kw) == status


def test_plan_paged_splits_is_the_tilegym_formula_on_the_longest_sequence():
    # hand-worked: est = 256 / 64 = 4, 32768 / 4 = 8192 -> L = 8192, 4 splits
    assert mla.plan_paged_splits(256, 64, 1, [1000] * 63 + [32768], 64) == (8192, 4)
    # est = 64, 4096 / 64 = 64 -> 128 (the page's floor), 32 splits
    assert mla.plan_paged_splits(256, 4, 1, [4096] * 4, 64) == (128, 32)
    # all lengths 0: the longest counts as 1 -> one split of 128
    assert mla.plan_paged_splits(1, 3, 2, [0, 0, 0], 32) == (128, 1)
    # est = 300 / 7 = 42, 70000 / 42 = 1666 -> 2048, ceil(70000 / 2048) = 35
    assert mla.plan_paged_splits(300, 7, 1, [5000, 129, 70000, 3, 8, 9, 10], 32) == (2048, 35)
    # the contiguous planner (pinned by the golden file) with S_kv = the longest sequence
    for cus in (1, 80, 256):
        for lens in ([1], [100, 7], [4096] * 4, [33, 70000, 5], [65536] * 64):
            assert mla.plan_paged_splits(cus, len(lens), 1, lens, 64) == \
                oracle.plan_contig(cus, len(lens), max(1, max(lens))), (cus, lens)


def test_plan_paged_splits_rejects():
    L = mla.lib()
    a, b = ctypes.c_int(), ctypes.c_int()
    sl = (ctypes.c_int32 * 2)(5, 6)
    p = ctypes.cast(sl, ctypes.c_void_p)
    assert L.mla_plan_paged_splits(256, 2, 1, None, 64, ctypes.byref(a), ctypes.byref(b)) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_plan_paged_splits(0, 2, 1, p, 64, ctypes.byref(a), ctypes.byref(b)) == mla.MLA_ERR_INVALID_ARG
    assert L.mla_plan_paged_splits(256, 2, 9, p, 64, ctypes.byref(a), ctypes.byref(b)) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_plan_paged_splits(256, 2, 1, p, 48, ctypes.byref(a), ctypes.byref(b)) == mla.MLA_ERR_UNSUPPORTED
    assert L.mla_plan_paged_splits(256, 2, 1, p, 64, None, ctypes.byref(b)) == mla.MLA_ERR_INVALID_ARG


def test_paged_splits_workspace_bytes():
    n = mla.paged_splits_workspace_bytes(64, 1, 128, 4)
    parts = 64 * 128 * 4
    assert n == -(-parts * 512 * 4 // 256) * 256 + -(-parts * 4 // 256) * 256
    assert n >= parts * oracle.workspace_floats_per_split(1, 1) * 4  # (D + 1) fp32 per split and head
    assert mla.paged_splits_workspace_bytes(0, 1, 128, 4) == 0
    assert mla.paged_splits_workspace_bytes(4, 1, 24, 4) == 0
    assert mla.paged_splits_workspace_bytes(4, 1, 128, 0) == 0


def _splits(**kw):
    a = dict(q=F, qpe=F, cache=F, fmt=1, kv_scale=1.0, num_pages=10, page_size=64, stride=64 * 576, bt=F, mb=4,
             sl=F, B=2, q_len=1, H=128, sm=0.07, L=128, ns=2, ws=F, ws_bytes=1 << 30, o=F, lse=F)
    a.update(kw)
    vp = ctypes.c_void_p
    return mla.lib().mla_paged_decode_splits(vp(a["q"]), vp(a["qpe"]), vp(a["cache"]), a["fmt"], a["kv_scale"],
                                             a["num_pages"], a["page_size"], a["stride"], vp(a["bt"]), a["mb"],
                                             vp(a["sl"]), a["B"], a["q_len"], a["H"], a["sm"], a["L"], a["ns"],
                                             vp(a["ws"]), a["ws_bytes"], vp(a["o"]), vp(a["lse"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), mla.MLA_ERR_INVALID_ARG),
    (dict(cache=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ws=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ws=F + 16), mla.MLA_ERR_INVALID_ARG),
    (dict(o=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lse=F + 2), mla.MLA_ERR_INVALID_ARG),
    (dict(fmt=4), mla.MLA_ERR_UNSUPPORTED),
    (dict(page_size=16), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_len=9), mla.MLA_ERR_UNSUPPORTED),
    (dict(H=24), mla.MLA_ERR_UNSUPPORTED),
    (dict(B=0), mla.MLA_ERR_INVALID_ARG),
    (dict(L=100), mla.MLA_ERR_INVALID_ARG),
    (dict(L=64), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=0), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=65536), mla.MLA_ERR_INVALID_ARG),
    (dict(ns=1), mla.MLA_ERR_INVALID_ARG),            # 1 x 128 tokens < 4 blocks x 64
    (dict(ws_bytes=1000), mla.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(kv_scale=0.0), mla.MLA_ERR_INVALID_ARG),
    (dict(sm=-1.0), mla.MLA_ERR_INVALID_ARG),
    (dict(stride=64 * 576 - 16), mla.MLA_ERR_INVALID_ARG),
])
def test_paged_decode_splits_rejects(kw, status):
    assert _splits(**kw) == status


def test_paged_decode_splits_workspace_boundary():
    need = mla.paged_splits_workspace_bytes(2, 1, 128, 2)
    assert _splits(ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
