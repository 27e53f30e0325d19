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
from gpu_util import TOL_LSE, TOL_O_BF16, TOL_O_QUANT, bf16_dev, check, host, i32_dev, max_err, say, u8_dev

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
    check("O", host(o), ro, tol)
    check("LSE", host(lse), rl, TOL_LSE)
