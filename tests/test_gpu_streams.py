"""The library keeps no state between calls (the no-alloc entry point aside): paged
decodes with their own workspaces run concurrently on two streams give bitwise the
results of the same calls run one after the other, and one workspace reused for calls
of different batches and split counts gives bitwise what a fresh workspace gives."""

import numpy as np
import pytest
import torch

import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import host, paged_device_inputs, say

pytestmark = pytest.mark.gpu


def _call(w, ns, workspace=None):
    d = paged_device_inputs(w)
    return mla.PagedCall(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                         w.kv_scale, w.sm_scale, num_splits=ns, workspace=workspace)


def _out(call):
    return host(call.o).copy(), host(call.lse).copy()


def test_two_streams_concurrently_match_serial():
    say("two streams, concurrent paged decodes")
    wa = gen.make_paged(B=8, H=128, q_len=1, lo=500, hi=3000, page_size=64, fmt=gen.FMT_FP8, seed=900)
    wb = gen.make_paged(B=5, H=64, q_len=2, lo=100, hi=2000, page_size=32, fmt=gen.FMT_NVFP4, seed=901)
    ca, cb = _call(wa, 96), _call(wb, 40)
    ca.run()
    cb.run()
    torch.cuda.synchronize()
    ref_a, ref_b = _out(ca), _out(cb)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for k in range(5):
        ca.o.zero_()
        cb.o.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            ca.run()
        with torch.cuda.stream(s2):
            cb.run()
        torch.cuda.synchronize()
        ga, gb = _out(ca), _out(cb)
        assert all(np.array_equal(x, y) for x, y in zip(ga, ref_a)), k
        assert all(np.array_equal(x, y) for x, y in zip(gb, ref_b)), k
    say("  5 concurrent rounds bitwise equal to the serial calls")


def test_reused_workspace_matches_fresh():
    say("one workspace across batches and split counts")
    cases = [
        (gen.make_paged(B=6, H=128, q_len=1, lo=1, hi=2500, page_size=64, fmt=gen.FMT_FP8, seed=910), 200),
        (gen.make_paged(B=3, H=32, q_len=2, lo=1, hi=1, page_size=32, fmt=gen.FMT_BF16, seed=911,
                        seq_lens=[0, 700, 3], max_blocks=23), 3),
        (gen.make_paged(B=6, H=128, q_len=1, lo=1, hi=2500, page_size=64, fmt=gen.FMT_FP8, seed=910), 7),
        (gen.make_paged(B=9, H=16, q_len=1, lo=0, hi=400, page_size=64, fmt=gen.FMT_NVFP4, seed=912), 64),
    ]
    n = max(mla.paged_workspace_bytes(w.B, w.q_len, w.H, ns) for w, ns in cases)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    for i, (w, ns) in enumerate(cases):
        if i % 2:
            ws.fill_(0xA5)  # arbitrary contents; even cases keep what the previous call left
        shared = _call(w, ns, workspace=ws)
        shared.run()
        fresh = _call(w, ns)
        fresh.run()
        torch.cuda.synchronize()
        a, b = _out(shared), _out(fresh)
        assert all(np.array_equal(x, y) for x, y in zip(a, b)), i
    say(f"  {len(cases)} calls on one workspace bitwise equal to fresh workspaces")
