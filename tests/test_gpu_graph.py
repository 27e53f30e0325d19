"""The paged decode under HIP graph capture: mla_paged_decode (caller workspace) and
mla_paged_decode_noalloc (the library's scratch array) enqueue only kernels (no
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
