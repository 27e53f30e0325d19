"""mla_paged_decode_noalloc (workspace in the library's own per-GPU scratch array)
against mla_paged_decode with a caller workspace: the same kernels, so the outputs must
be bit-identical; two calls in a row, the second on a smaller problem, so the second
runs on what the first left in the scratch array.  Both are also checked against the
oracle."""

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import TOL_LSE, TOL_O_QUANT, check, check_o, host, paged_device_inputs, say

pytestmark = pytest.mark.gpu


def _both(w):
    d = paged_device_inputs(w)
    args = (d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride, w.kv_scale,
            w.sm_scale)
    o1, l1 = mla.paged_decode(*args)
    o2, l2 = mla.paged_decode_noalloc(*args)
    torch.cuda.synchronize()
    return host(o1), host(l1), host(o2), host(l2)


def test_noalloc_matches_workspace_path_twice():
    cases = [dict(B=8, H=128, q_len=2, lo=100, hi=3000, page_size=64, fmt=gen.FMT_FP8, seed=301),
             dict(B=3, H=32, q_len=1, lo=1, hi=200, page_size=32, fmt=gen.FMT_NVFP4, seed=302)]
    for c in cases:
        say(f"noalloc {c}")
        w = gen.make_paged(**c, poison_tail=True)
        o1, l1, o2, l2 = _both(w)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2, equal_nan=True)
        q, qpe = w.q_f64()
        ro, rl = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                     w.block_tables, w.seq_lens, w.sm_scale)
        check_o("noalloc O", o2, ro, TOL_O_QUANT)
        check("noalloc LSE", l2, rl, TOL_LSE)


def test_noalloc_rejects_problems_beyond_the_scratch():
    w = gen.make_paged(B=2, H=128, q_len=8, lo=10, hi=20, page_size=64, fmt=gen.FMT_FP8, seed=303)
    d = paged_device_inputs(w)
    need = mla.paged_workspace_bytes(w.B, w.q_len, w.H, 2000)
    assert need > mla.MLA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MlaError) as e:
        mla.paged_decode_noalloc(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                                 w.kv_scale, w.sm_scale, num_splits=2000)
    assert e.value.status == mla.MLA_ERR_SCRATCH_LIMIT
