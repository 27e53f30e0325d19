"""The paged decode's two launches on their own (mla_paged_decode_partials, then
mla_paged_combine), as the benchmark times them: the split plan the decode launch
builds on the device (seg_first, seg_last, info[0] in the workspace) is compared
bit-exactly with the Python mirror of the plan, every live partial slot's O_j and lse_j
with the oracle over that slot's token range, and the combine's output bit-exactly with
mla_paged_decode's."""

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
import plan_mirror as pm
from workloads import gen
from gpu_util import TOL_LSE, TOL_O_BF16, TOL_O_QUANT, check, check_o, host, paged_device_inputs, say

pytestmark = pytest.mark.gpu


def _run_partials(w, ns):
    d = paged_device_inputs(w)
    call = mla.PagedCall(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                         w.kv_scale, w.sm_scale, num_splits=ns)
    call.partials()
    torch.cuda.synchronize()
    ws = call.workspace.cpu().numpy().copy()
    o, lse = call.combine()
    torch.cuda.synchronize()
    o_c, l_c = host(o).copy(), host(lse).copy()
    o2, l2 = call.run()  # both launches through mla_paged_decode
    torch.cuda.synchronize()
    return ws, o_c, l_c, host(o2), host(l2)


def _parse(ws, B, q_len, H, ns):
    L = pm.workspace_layout(B, q_len, H, ns)
    assert ws.size >= L["total"]
    rows, slots = L["rows"], L["slots"]
    o_part = ws[L["o_off"]:L["o_off"] + slots * rows * 512 * 4].view(np.float32).reshape(slots, rows, 512)
    lse_part = ws[L["lse_off"]:L["lse_off"] + slots * rows * 4].view(np.float32).reshape(slots, rows)
    first = ws[L["first_off"]:L["first_off"] + 4 * B].view(np.int32)
    last = ws[L["last_off"]:L["last_off"] + 4 * B].view(np.int32)
    info = ws[L["info_off"]:L["info_off"] + 256].view(np.int32)
    return o_part, lse_part, first, last, info


def _check_plan_and_slots(w, ns, max_slots=None, seed=0):
    ws, o_c, l_c, o_r, l_r = _run_partials(w, ns)
    # the separate launches give exactly what mla_paged_decode gives
    assert np.array_equal(o_c, o_r) and np.array_equal(l_c, l_r)
    max_len = w.max_blocks * w.page_size
    segs, first, last, W = pm.plan(w.seq_lens, max_len, ns, w.q_len, tile=pm.tile_tokens(w.fmt))
    o_part, lse_part, dfirst, dlast, info = _parse(ws, w.B, w.q_len, w.H, ns)
    assert int(info[0]) == W
    for b in range(w.B):
        if first[b] >= 0:  # requests without tiles have no descriptors
            assert (int(dfirst[b]), int(dlast[b])) == (first[b], last[b]), b
    say(f"  plan: {len(segs)} segments over {ns} ranges, W={W}: descriptors bit-exact")
    # every live slot against the oracle over its token range
    pick = segs
    if max_slots is not None and len(segs) > max_slots:
        rng = np.random.default_rng(seed)
        pick = [segs[i] for i in sorted(rng.choice(len(segs), max_slots, replace=False))]
    q, qpe = w.q_f64()
    tol = TOL_O_BF16 if w.fmt == gen.FMT_BF16 else TOL_O_QUANT
    eo = el = 0.0
    kv_cache = {}
    for s in pick:
        n = int(w.seq_lens[s.b])
        if s.b not in kv_cache:
            kv_cache = {s.b: oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                                   w.block_tables[s.b], n)}
        kv = kv_cache[s.b]
        vis = np.repeat(oracle.visible_counts(n, w.q_len), w.H)
        qf = np.concatenate([q[s.b], qpe[s.b]], axis=-1).reshape(w.q_len * w.H, 576)
        ro, rl = oracle.attend_range(qf, kv, vis, w.sm_scale, s.t0, s.t1)
        go, gl = o_part[s.slot].astype(np.float64), lse_part[s.slot].astype(np.float64)
        live = np.isfinite(rl)
        assert np.array_equal(np.isneginf(gl), ~live), s  # rows that see nothing: -inf
        eo = max(eo, float(np.abs(go[live] - ro[live]).max()) if live.any() else 0.0)
        el = max(el, float(np.abs(gl[live] - rl[live]).max()) if live.any() else 0.0)
    say(f"  {len(pick)} slots: O_j max|d|={eo:.3e} (tol {tol:.0e}), lse_j max|d|={el:.3e} (tol {TOL_LSE:.0e})")
    assert eo <= tol and el <= TOL_LSE
    return o_c, l_c


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("ns", [1, 3, 16, 64, 300])
def test_partials_plan_and_slots_random(seed, ns):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(2, 12))
    lens = rng.integers(0, 900, size=B)
    lens[rng.random(B) < 0.2] = 0
    lens[0] = max(int(lens[0]), 1)
    fmt = (gen.FMT_FP8, gen.FMT_BF16, gen.FMT_NVFP4)[seed]
    q_len = 1 + seed % 2
    H = (128, 32, 64)[seed]
    say(f"partials plan seed={seed} ns={ns} B={B} fmt={fmt} q_len={q_len} H={H}")
    w = gen.make_paged(B=B, H=H, q_len=q_len, lo=1, hi=1, page_size=(64, 32, 64)[seed], fmt=fmt,
                       seed=200 + seed, seq_lens=lens.tolist(), poison_tail=True,
                       max_blocks=int(-(-max(lens) // 32)) + 1)
    _check_plan_and_slots(w, ns)


def test_partials_headline_full_size():
    """The benchmark workload and launch configuration: descriptors bit-exact, 24 sampled
    slots against the oracle, and the combine against the whole batch's oracle output
    for three requests."""
    say("partials headline full size")
    w = gen.make_workload("paged_fp8_b64_h128_s1k_32k")
    ns = mla.plan_paged(256, w.B, w.q_len, w.H)
    o, lse = _check_plan_and_slots(w, ns, max_slots=24, seed=5)
    pick = [0, 31, 63]
    ro, rl = oracle.paged_decode(*w.q_f64(), w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                 w.block_tables, w.seq_lens, w.sm_scale, requests=pick)
    check_o("combine O", o[pick], ro, TOL_O_QUANT)
    check("combine LSE", lse[pick], rl, TOL_LSE)


@pytest.mark.parametrize("B,fmt", [(1000, gen.FMT_BF16), (4096, gen.FMT_FP8)])
def test_partials_plan_many_requests(B, fmt):
    """Batches larger than the workgroup (each thread of the device prefix scan sums 4 or
    16 requests), short and empty requests, many segments per range (the largest batch the
    library takes): descriptors bit-exact against the mirror, sampled slots and sampled
    requests' outputs against the oracle."""
    rng = np.random.default_rng(500 + B)
    lens = rng.integers(0, 60, size=B)
    lens[rng.random(B) < 0.1] = 0
    lens[0] = 1
    say(f"partials plan B={B} fmt={fmt}, {int((lens > 0).sum())} non-empty requests")
    w = gen.make_paged(B=B, H=16, q_len=1, lo=0, hi=60, page_size=32, fmt=fmt, seed=600 + B,
                       seq_lens=lens.tolist(), max_blocks=2, poison_tail=True)
    ns = mla.plan_paged(256, w.B, w.q_len, w.H)
    o, lse = _check_plan_and_slots(w, ns, max_slots=64, seed=B)
    pick = sorted(set(rng.choice(B, 64, replace=False).tolist()) | {0, B - 1})
    ro, rl = oracle.paged_decode(*w.q_f64(), w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                 w.block_tables, w.seq_lens, w.sm_scale, requests=pick)
    check_o(f"O ({len(pick)} requests)", o[pick], ro, TOL_O_BF16 if fmt == gen.FMT_BF16 else TOL_O_QUANT)
    check(f"LSE ({len(pick)} requests)", lse[pick], rl, TOL_LSE)
