"""The decodes under HIP graph capture: mla_paged_decode (caller workspace),
mla_paged_decode_noalloc (the library's scratch array), the contiguous decode with its
combine, and the paged decode with fixed-length splits enqueue only kernels (no
allocation, no memset), so a captured call replays the same work.  Each graph is replayed
several times, with eager work and synchronisation between the replays and the outputs
cleared before each, and every replay must equal the eager result bit for bit."""

import numpy as np
import pytest
import torch

import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import host, paged_device_inputs, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("noalloc", [False, True])
def test_paged_decode_replays_bitwise(noalloc):
    say(f"graph replay noalloc={noalloc}")
    w = gen.make_paged(B=6, H=128, q_len=2, lo=1, hi=2500, page_size=64, fmt=gen.FMT_FP8, seed=800, poison_tail=True)
    d = paged_device_inputs(w)
    args = (d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride, w.kv_scale,
            w.sm_scale)
    ns = mla.plan_paged(mla.device_num_cus(0), w.B, w.q_len, w.H)
    o = torch.empty((w.B, w.q_len, w.H, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device="cuda:0")
    if noalloc:
        run = lambda: mla.paged_decode_noalloc(*args, num_splits=ns, o=o, lse=lse)
    else:
        ws = mla.paged_workspace(w.B, w.q_len, w.H, ns, torch.device("cuda:0"))
        run = lambda: mla.paged_decode(*args, num_splits=ns, workspace=ws, o=o, lse=lse)
    run()
    torch.cuda.synchronize()
    ref_o, ref_l = host(o).copy(), host(lse).copy()
    g = _capture(run)
    scratch = torch.ones(1 << 20, device="cuda:0")
    for k in range(4):
        o.zero_()
        lse.zero_()
        scratch.mul_(1.0001)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(o), ref_o) and np.array_equal(host(lse), ref_l), k
    say("  4 replays bitwise equal to the eager call")


def _replay_check(run, outs):
    run()
    torch.cuda.synchronize()
    refs = [host(t).copy() for t in outs]
    g = _capture(run)
    scratch = torch.ones(1 << 20, device="cuda:0")
    for k in range(4):
        for t in outs:
            t.zero_()
        scratch.mul_(1.0001)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(np.array_equal(host(t), r) for t, r in zip(outs, refs)), k


def test_contig_decode_and_combine_replay_bitwise():
    say("graph replay: contiguous decode + combine")
    c = gen.make_contig(3, 128, 1500, seed=810)
    q, qpe, kv, kpe = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
                       for a in (c.q, c.qpe, c.kv, c.kpe))
    L, ns = mla.plan_contig(mla.device_num_cus(0), c.B, c.S)
    op = torch.empty((c.B, c.H, ns, 512), dtype=torch.float32, device="cuda:0")
    lp = torch.empty((c.B, c.H, ns), dtype=torch.float32, device="cuda:0")
    o = torch.empty((c.B, c.H, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((c.B, c.H), dtype=torch.float32, device="cuda:0")

    def run():
        mla.decode_splitkv(q, qpe, kv, kpe, c.sm_scale, L, o_part=op, lse_part=lp)
        mla.splitkv_combine(op, lp, o=o, lse=lse)

    _replay_check(run, [op, lp, o, lse])
    say("  4 replays bitwise equal to the eager calls")


def test_paged_fixed_splits_replay_bitwise():
    say("graph replay: paged decode with fixed-length splits")
    w = gen.make_paged(B=5, H=64, q_len=2, lo=1, hi=3000, page_size=64, fmt=gen.FMT_NVFP4, seed=811,
                       poison_tail=True)
    d = paged_device_inputs(w)
    L, ms = mla.plan_paged_splits(mla.device_num_cus(0), w.B, w.q_len, w.seq_lens.tolist(), w.page_size)
    ms = max(ms, -(-(w.max_blocks * w.page_size) // L))
    ws = torch.empty(mla.paged_splits_workspace_bytes(w.B, w.q_len, w.H, ms), dtype=torch.uint8, device="cuda:0")
    o = torch.empty((w.B, w.q_len, w.H, 512), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device="cuda:0")
    run = lambda: mla.paged_decode_splits(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size,
                                          w.page_stride, w.kv_scale, w.sm_scale, kv_len_per_split=L, max_splits=ms,
                                          workspace=ws, o=o, lse=lse)
    _replay_check(run, [o, lse])
    say(f"  L={L}, {ms} splits: 4 replays bitwise equal to the eager call")
