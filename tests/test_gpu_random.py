"""Randomised GPU parity: seeded draws over cache format, head count, query count, page
size and stride, batch, lengths (including empty requests), sliding window, sinks and
split count, each compared with the oracle on every output.  Each case prints its
parameters before it runs."""

import os

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import TOL_LSE, TOL_O_BF16, TOL_O_QUANT, bf16_dev, check, check_o, host, i32_dev, max_err, say, u8_dev

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    fmt = int(rng.choice([gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4, oracle.FMT_FP8_QFP8]))
    H = int(rng.choice([16, 32, 48, 64, 128]))
    q_len = int(rng.integers(1, 9))
    page_size = int(rng.choice([32, 64]))
    B = int(rng.integers(1, 7))
    seq = rng.integers(0, 700, size=B)
    seq[rng.random(B) < 0.15] = 0
    window = int(rng.choice([0, 0, int(rng.integers(1, 500))]))
    with_sinks = bool(rng.random() < 0.5)
    ns = None if rng.random() < 0.4 else int(rng.integers(1, 41))
    pad = int(rng.choice([0, 16, 48]))
    return dict(fmt=fmt, H=H, q_len=q_len, page_size=page_size, B=B, seq=[int(x) for x in seq], window=window,
                sinks=with_sinks, num_splits=ns, pad=pad, seed=seed)


# MLA_RANDOM_CASES widens the sweep (default 24 cases)
@pytest.mark.parametrize("seed", range(int(os.environ.get("MLA_RANDOM_CASES", "24"))))
def test_random_paged_case_matches_oracle(seed):
    c = _case(seed)
    say(f"random case {c}")
    base_fmt = gen.FMT_FP8 if c["fmt"] == oracle.FMT_FP8_QFP8 else c["fmt"]
    stride = c["page_size"] * oracle.page_row_bytes(base_fmt) + c["pad"]
    mb = max(1, max(-(-n // c["page_size"]) for n in c["seq"]) + 1)
    w = gen.make_paged(B=c["B"], H=c["H"], q_len=c["q_len"], lo=0, hi=700, page_size=c["page_size"], fmt=base_fmt,
                       seed=9100 + seed, seq_lens=c["seq"], max_blocks=mb, page_stride=stride, poison_tail=True)
    w.fmt = c["fmt"]
    sinks = (np.random.default_rng(seed).standard_normal(c["H"]) * 2).astype(np.float32) if c["sinks"] else None
    q, qpe = w.q_f64()
    ro, rl = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables,
                                 w.seq_lens, w.sm_scale, window=c["window"],
                                 sinks=None if sinks is None else sinks.astype(np.float64))
    o, lse = mla.paged_decode(bf16_dev(w.q), bf16_dev(w.qpe), u8_dev(w.cache), w.fmt, i32_dev(w.block_tables),
                              i32_dev(w.seq_lens), w.page_size, w.page_stride, w.kv_scale, w.sm_scale,
                              num_splits=c["num_splits"], window=c["window"],
                              sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV))
    torch.cuda.synchronize()
    tol = TOL_O_BF16 if base_fmt == gen.FMT_BF16 else TOL_O_QUANT
    check_o("O", host(o), ro, tol)
    check("LSE", host(lse), rl, TOL_LSE)


def _splits_case(seed):
    rng = np.random.default_rng(9500 + seed)
    fmt = int(rng.choice([gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4, oracle.FMT_FP8_QFP8]))
    H = int(rng.choice([16, 32, 48, 64, 128]))
    q_len = int(rng.integers(1, 9))
    page_size = int(rng.choice([32, 64]))
    B = int(rng.integers(1, 7))
    seq = rng.integers(0, 900, size=B)
    seq[rng.random(B) < 0.15] = 0
    L = None if rng.random() < 0.3 else int(rng.choice([128, 256, 512]))
    extra = int(rng.integers(0, 3))  # splits beyond the ones the table needs
    pad = int(rng.choice([0, 16, 48]))
    return dict(fmt=fmt, H=H, q_len=q_len, page_size=page_size, B=B, seq=[int(x) for x in seq], L=L, extra=extra,
                pad=pad, seed=seed)


@pytest.mark.parametrize("seed", range(int(os.environ.get("MLA_RANDOM_CASES", "24")) // 2))
def test_random_fixed_splits_case_matches_oracle(seed):
    """The fixed-length split interface on random batches: final O / LSE and every split's
    partial (workspace read back) against the oracle's fixed-split partials."""
    c = _splits_case(seed)
    say(f"random fixed-split case {c}")
    base_fmt = gen.FMT_FP8 if c["fmt"] == oracle.FMT_FP8_QFP8 else c["fmt"]
    stride = c["page_size"] * oracle.page_row_bytes(base_fmt) + c["pad"]
    mb = max(1, max(-(-n // c["page_size"]) for n in c["seq"]) + 1)
    w = gen.make_paged(B=c["B"], H=c["H"], q_len=c["q_len"], lo=0, hi=900, page_size=c["page_size"], fmt=base_fmt,
                       seed=9600 + seed, seq_lens=c["seq"], max_blocks=mb, page_stride=stride, poison_tail=True)
    w.fmt = c["fmt"]
    L = c["L"]
    if L is None:
        L, _ = mla.plan_paged_splits(mla.device_num_cus(0), w.B, w.q_len, w.seq_lens.tolist(), w.page_size)
    ns = -(-mb * c["page_size"] // L) + c["extra"]
    nbytes = mla.paged_splits_workspace_bytes(w.B, w.q_len, w.H, ns)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    o, lse, _, _ = mla.paged_decode_splits(bf16_dev(w.q), bf16_dev(w.qpe), u8_dev(w.cache), w.fmt,
                                           i32_dev(w.block_tables), i32_dev(w.seq_lens), w.page_size, w.page_stride,
                                           w.kv_scale, w.sm_scale, kv_len_per_split=L, max_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    q, qpe = w.q_f64()
    args = (q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables, w.seq_lens, w.sm_scale)
    ro, rl = oracle.paged_decode(*args)
    rop, rlp = oracle.paged_decode_split_partials(*args, L, ns)
    tol = TOL_O_BF16 if base_fmt == gen.FMT_BF16 else TOL_O_QUANT
    check_o("O", host(o), ro, tol)
    check("LSE", host(lse), rl, TOL_LSE)
    parts = w.B * w.q_len * w.H * ns
    lse_off = -(-parts * 512 * 4 // 256) * 256
    op = host(ws[:parts * 512 * 4].view(torch.float32)).reshape(rop.shape)
    lp = host(ws[lse_off:lse_off + parts * 4].view(torch.float32)).reshape(rlp.shape)
    check("lse_part", lp, rlp, TOL_LSE)
    live = np.isfinite(rlp)
    check("o_part", op[live], rop[live], tol)


@pytest.mark.parametrize("seed", range(int(os.environ.get("MLA_RANDOM_CASES", "24")) // 2))
def test_random_contig_case_matches_oracle(seed):
    """The contiguous op on random shapes (any number of (request, split) items, so every
    placement of the items over the XCDs' id ranges): partials and combined output."""
    rng = np.random.default_rng(9700 + seed)
    B = int(rng.integers(1, 10))
    H = int(rng.choice([16, 32, 48, 64, 80, 128]))
    S = int(rng.integers(1, 2500))
    L = None if rng.random() < 0.3 else int(rng.choice([128, 256, 512, 1024]))
    say(f"random contiguous case B={B} H={H} S={S} L={L}")
    c = gen.make_contig(B, H, S, seed=9800 + seed)
    op, lp, L = mla.decode_splitkv(bf16_dev(c.q), bf16_dev(c.qpe), bf16_dev(c.kv), bf16_dev(c.kpe), c.sm_scale, L)
    o, lse = mla.splitkv_combine(op, lp)
    torch.cuda.synchronize()
    q, qpe, kv, kpe = c.f64()
    rop, rlp = oracle.contig_decode_splitkv(q, qpe, kv, kpe, c.sm_scale, L)
    ro, rl = oracle.contig_decode(q, qpe, kv, kpe, c.sm_scale)
    check("o_part", host(op), rop, TOL_O_BF16)
    check("lse_part", host(lp), rlp, TOL_LSE)
    check_o("O", host(o), ro, TOL_O_BF16)
    check("LSE", host(lse), rl, TOL_LSE)
