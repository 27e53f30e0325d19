"""GPU parity of the paged decode with fixed-length splits (mla_paged_decode_splits):
the final O / LSE against the float64 oracle, and every split's partial O_j / lse_j in
the caller's workspace against the oracle's fixed-split partials.  Split j of a request
covers its tokens [j*L, (j+1)*L); splits past a request's length are empty."""

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import TOL_LSE, TOL_O_BF16, TOL_O_QUANT, check, check_o, host, paged_device_inputs, say

pytestmark = pytest.mark.gpu


def _tol_o(fmt):
    return TOL_O_BF16 if fmt == gen.FMT_BF16 else TOL_O_QUANT


def _run(w, L=None, ns=None):
    """Run with a workspace filled with 0xFF bytes (NaN as f32) so an unwritten partial
    that the combine reads shows up.  Returns O, LSE, L, NS and the partials."""
    d = paged_device_inputs(w)
    if L is None:
        L, _ = mla.plan_paged_splits(mla.device_num_cus(0), w.B, w.q_len, w.seq_lens.tolist(), w.page_size)
    if ns is None:
        ns = -(-w.max_blocks * w.page_size // L)
    nbytes = mla.paged_splits_workspace_bytes(w.B, w.q_len, w.H, ns)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    o, lse, L2, ns2 = mla.paged_decode_splits(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size,
                                              w.page_stride, w.kv_scale, w.sm_scale, kv_len_per_split=L,
                                              max_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert (L2, ns2) == (L, ns)
    parts = w.B * w.q_len * w.H * ns
    lse_off = -(-parts * 512 * 4 // 256) * 256
    op = ws[:parts * 512 * 4].view(torch.float32).reshape(w.B, w.q_len, w.H, ns, 512)
    lp = ws[lse_off:lse_off + parts * 4].view(torch.float32).reshape(w.B, w.q_len, w.H, ns)
    return host(o), host(lse), L, ns, host(op), host(lp)


def _refs(w, L, ns, requests=None):
    q, qpe = w.q_f64()
    bs = list(range(w.B)) if requests is None else list(requests)
    args = (q[bs], qpe[bs], w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables[bs],
            w.seq_lens[bs], w.sm_scale)
    ro, rl = oracle.paged_decode(*args)
    rop, rlp = oracle.paged_decode_split_partials(*args, L, ns)
    return ro, rl, rop, rlp


def _check_all(w, got, refs, what=""):
    o, lse, L, ns, op, lp = got
    ro, rl, rop, rlp = refs
    check_o(f"o {what}", o, ro, _tol_o(w.fmt))
    check(f"lse {what}", lse, rl, TOL_LSE)
    check(f"lse_part {what}", lp, rlp, TOL_LSE)
    live = np.isfinite(rlp)
    check(f"o_part {what}", op[live], rop[live], _tol_o(w.fmt))


def _workload(fmt, q_len, page_size, seed):
    w = gen.make_paged(B=5, H=128, q_len=q_len, lo=1, hi=1, page_size=page_size,
                       fmt=gen.FMT_FP8 if fmt == oracle.FMT_FP8_QFP8 else fmt, seed=seed,
                       seq_lens=[0, 63, 290, 129, 1], max_blocks=1024 // page_size, poison_tail=True)
    w.fmt = fmt  # the FP8-query format reads the FP8 format's pages
    return w


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4, oracle.FMT_FP8_QFP8])
@pytest.mark.parametrize("q_len", [1, 2])
@pytest.mark.parametrize("page_size", [32, 64])
def test_paged_splits_match_oracle(fmt, q_len, page_size):
    """Ragged lengths with an empty request, a one-token one and one whose last split holds
    one token (q_len 2: query 0 sees none of it); L from the planner, the
    smallest L (eight splits), an L with trailing empty splits, and one split."""
    say(f"paged splits fmt={fmt} q_len={q_len} page={page_size}")
    w = _workload(fmt, q_len, page_size, seed=200 + 10 * fmt + q_len + page_size)
    for L, ns in ((None, None), (128, None), (256, 6), (1024, 1)):
        got = _run(w, L, ns)
        _check_all(w, got, _refs(w, got[2], got[3]), f"L={got[2]} ns={got[3]}")
        assert (got[0][0] == 0).all() and np.isneginf(got[1][0]).all()  # the empty request


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
@pytest.mark.parametrize("H,q_len", [(16, 1), (48, 2), (64, 4), (128, 8)])
def test_paged_splits_head_and_query_counts(fmt, H, q_len):
    say(f"paged splits fmt={fmt} H={H} q_len={q_len}")
    w = gen.make_paged(B=3, H=H, q_len=q_len, lo=8, hi=400, page_size=64, fmt=fmt, seed=230 + H + q_len,
                       max_blocks=8)
    got = _run(w, 128)
    _check_all(w, got, _refs(w, got[2], got[3]))


def test_paged_splits_one_long_request_many_splits():
    """A 16000-token request beside a short one at L = 128: 125 splits per row, merged in
    two rounds of 64 by the combine; the short request's 124 empty splits add nothing."""
    say("paged splits one long request")
    w = gen.make_paged(B=2, H=16, q_len=1, lo=1, hi=1, page_size=64, fmt=gen.FMT_FP8, seed=240,
                       seq_lens=[16000, 40], max_blocks=250)
    got = _run(w, 128)
    assert got[3] == 125
    _check_all(w, got, _refs(w, 128, 125))


def test_paged_splits_agree_with_the_planned_path_and_repeat_bitwise():
    """Both paged entry points compute the same attention: on the same inputs their
    results agree to the tolerance, and a repeated call is bit-identical."""
    say("paged splits vs planned path")
    w = gen.make_paged(B=6, H=128, q_len=1, lo=1, hi=3000, page_size=64, fmt=gen.FMT_FP8, seed=250)
    d = paged_device_inputs(w)
    o1, l1 = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                              w.kv_scale, w.sm_scale)
    a = _run(w)
    b = _run(w)
    torch.cuda.synchronize()
    check_o("o vs planned", a[0], host(o1), TOL_O_QUANT)
    check("lse vs planned", a[1], host(l1), TOL_LSE)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_paged_splits_fp8_b64_h128_full_size():
    """The FP8 benchmark pages (64 requests, 1k-32k tokens, 128 heads) with the planner's
    L: every request's output, and the partials of the shortest, the longest and two
    middle requests."""
    say("paged splits fp8 b64 h128 full size")
    w = gen.make_workload("paged_fp8_b64_h128_s1k_32k")
    got = _run(w)
    o, lse, L, ns, op, lp = got
    say(f"  L={L} ns={ns}")
    assert np.isfinite(o).all()
    ro, rl = oracle.paged_decode(*w.q_f64(), w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                 w.block_tables, w.seq_lens, w.sm_scale)
    check_o("O (64 requests)", o, ro, TOL_O_QUANT)
    check("LSE (64 requests)", lse, rl, TOL_LSE)
    order = np.argsort(w.seq_lens)
    pick = sorted({int(order[0]), int(order[21]), int(order[42]), int(order[63])})
    q, qpe = w.q_f64()
    rop, rlp = oracle.paged_decode_split_partials(q[pick], qpe[pick], w.cache, w.fmt, w.kv_scale, w.page_size,
                                                  w.page_stride, w.block_tables[pick], w.seq_lens[pick], w.sm_scale,
                                                  L, ns)
    check("lse_part (4 requests)", lp[pick], rlp, TOL_LSE)
    live = np.isfinite(rlp)
    check("o_part (4 requests)", op[pick][live], rop[live], TOL_O_QUANT)
