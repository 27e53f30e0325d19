"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, element by
element on the same seeded inputs.  Small cases span several tiles and ragged tails;
the full-size workloads compare sampled requests (every head and query of each sampled
request) that the oracle computes one by one."""

import math

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import (TOL_LSE, TOL_O_BF16, TOL_O_QUANT, bf16_dev, check, check_o, host, i32_dev, max_err,
                      paged_device_inputs, say, u8_dev)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _contig_run(c, L):
    q, qpe, kv, kpe = (bf16_dev(a) for a in (c.q, c.qpe, c.kv, c.kpe))
    op, lp, L = mla.decode_splitkv(q, qpe, kv, kpe, c.sm_scale, L)
    o, lse = mla.splitkv_combine(op, lp)
    torch.cuda.synchronize()
    return host(op), host(lp), host(o), host(lse), L


@pytest.mark.parametrize("B,H,S,L", [
    (1, 16, 256, 128),     # tiny contiguous workload: 2 splits (one tile per wavefront, one merge round)
    (2, 32, 300, 128),     # ragged last split (44 tokens, partial tile; two merge rounds, two idle wavefronts)
    (3, 16, 33, 128),      # one full tile and one token: two wavefronts idle
    (2, 16, 4096, 256),    # few heads, 8 tiles per split: the tile loop with shared dims
    (1, 48, 200, 128),     # rows not a multiple of 32: one wave half idle, two waves idle
    (2, 128, 1000, 256),   # full head group, 4 splits, ragged
    (3, 64, 129, 128),     # one token in the last split
    (2, 16, 4096, 1024),   # few heads over long splits: 4 wavefronts share each row block
    (2, 32, 65, 128),      # 3 tiles in one split, all loaded at once, ragged
    (1, 96, 500, 128),     # three row blocks, one wavefront idle
])
def test_contig_splitkv_matches_oracle(B, H, S, L):
    say(f"contig B={B} H={H} S={S} L={L}")
    c = gen.make_contig(B, H, S, seed=7 + B + H + S)
    op, lp, o, lse, _ = _contig_run(c, L)
    q, qpe, kv, kpe = c.f64()
    rop, rlp = oracle.contig_decode_splitkv(q, qpe, kv, kpe, c.sm_scale, L)
    ro, rl = oracle.contig_decode(q, qpe, kv, kpe, c.sm_scale)
    check("op", op, rop, TOL_O_BF16)
    check("lp", lp, rlp, TOL_LSE)
    check_o("o", o, ro, TOL_O_BF16)
    check("lse", lse, rl, TOL_LSE)


def test_contig_b4_h16_s4096_full_size():
    say("contig_b4_h16_s4096 full size")
    c = gen.make_workload("contig_b4_h16_s4096")
    L, ns = mla.plan_contig(256, c.B, c.S)
    assert (L, ns) == (128, 32)
    op, lp, o, lse, _ = _contig_run(c, L)
    q, qpe, kv, kpe = c.f64()
    ro, rl = oracle.contig_decode(q, qpe, kv, kpe, c.sm_scale)
    check_o("o", o, ro, TOL_O_BF16)
    check("lse", lse, rl, TOL_LSE)
    rop, rlp = oracle.contig_decode_splitkv(q[:1], qpe[:1], kv[:1], kpe[:1], c.sm_scale, L)
    check("op[:1]", op[:1], rop, TOL_O_BF16)
    check("lp[:1]", lp[:1], rlp, TOL_LSE)


def test_contig_b32_h128_s8192_full_size():
    """Every request of the contiguous B=32 H=128 workload, final and per-split outputs."""
    say("contig_b32_h128_s8192 full size, all 32 requests")
    c = gen.make_workload("contig_b32_h128_s8192")
    L, ns = mla.plan_contig(256, c.B, c.S)
    assert (L, ns) == (1024, 8)
    op, lp, o, lse, _ = _contig_run(c, L)
    q, qpe, kv, kpe = c.f64()
    eo = el = epo = epl = 0.0
    for b in range(c.B):
        ro, rl = oracle.contig_decode(q[b:b + 1], qpe[b:b + 1], kv[b:b + 1], kpe[b:b + 1], c.sm_scale)
        eo, el = max(eo, max_err(o[b:b + 1], ro)), max(el, max_err(lse[b:b + 1], rl))
        rop, rlp = oracle.contig_decode_splitkv(q[b:b + 1], qpe[b:b + 1], kv[b:b + 1], kpe[b:b + 1], c.sm_scale, L)
        epo, epl = max(epo, max_err(op[b:b + 1], rop)), max(epl, max_err(lp[b:b + 1], rlp))
    say(f"  O max|d|={eo:.3e} LSE {el:.3e} O_j {epo:.3e} lse_j {epl:.3e} (tol {TOL_O_BF16:.0e} / {TOL_LSE:.0e})")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE and epo <= TOL_O_BF16 and epl <= TOL_LSE


def test_contig_requests_past_4gib_periodic_cache():
    """Two requests of 4,198,400 tokens (a 9.7 GB cache; request 1's latent rows start past
    4 GiB), each cache a 4096-token random block repeated 1025 times.  Attention over m
    copies of a block equals attention over one block with ln m added to the LSE, so the
    oracle runs on one block: every split (16 copies, the last one copy) and the merged
    output are checked against it."""
    say("contig requests past 4 GiB, periodic cache")
    P, reps = 4096, 1025
    c = gen.make_contig(2, 128, P, seed=91)
    q, qpe, kv, kpe = (bf16_dev(a) for a in (c.q, c.qpe, c.kv, c.kpe))
    kv_big, kpe_big = kv.repeat(1, reps, 1), kpe.repeat(1, reps, 1)
    S = P * reps
    assert kv_big.shape[1] == S and S * 512 * 2 > 2 ** 32
    del kv, kpe
    op, lp, L = mla.decode_splitkv(q, qpe, kv_big, kpe_big, c.sm_scale)
    o, lse = mla.splitkv_combine(op, lp)
    torch.cuda.synchronize()
    ns = -(-S // L)
    assert (L, ns) == (65536, 65)
    del kv_big, kpe_big
    torch.cuda.empty_cache()
    qd, qped, kvd, kped = c.f64()
    ro, rl = oracle.contig_decode(qd, qped, kvd, kped, c.sm_scale)  # one block: [B, H, 512], [B, H]
    copies = np.array([L // P] * (ns - 1) + [(S - (ns - 1) * L) // P], dtype=np.float64)
    check("op", host(op), np.broadcast_to(ro[:, :, None, :], op.shape), TOL_O_BF16)
    check("lp", host(lp), rl[:, :, None] + np.log(copies)[None, None, :], TOL_LSE)
    check_o("o", host(o), ro, TOL_O_BF16)
    check("lse", host(lse), rl + math.log(reps), TOL_LSE)


def test_contig_zero_query_is_mean_of_latent():
    say("contig zero query")
    c = gen.make_contig(2, 16, 333, seed=3, zero_q=True)
    _, _, o, lse, _ = _contig_run(c, 128)
    kv = gen.bf16_bits_to_f32(c.kv).astype(np.float64)
    mean = kv.mean(axis=1)  # [B, 512]
    assert np.abs(o - mean[:, None, :]).max() <= TOL_O_BF16
    assert np.abs(lse - math.log(333)).max() <= TOL_LSE


def test_contig_run_to_run_bitwise_stable():
    say("contig determinism")
    c = gen.make_contig(2, 128, 700, seed=5)
    a = _contig_run(c, 256)
    b = _contig_run(c, 256)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("R,NS", [(37, 9), (11, 150), (13, 8), (10, 33)])
def test_combine_matches_oracle_with_empty_splits(R, NS):
    """Up to 8 partials a row takes one wavefront with every load issued at once; more take
    a workgroup per row, whose four wavefronts merge every fourth partial in batches of 8
    (NS = 150: five batches each, the last ragged) and then merge their results."""
    say(f"combine generic R={R} NS={NS}")
    rng = np.random.default_rng(4 + NS)
    op = rng.standard_normal((R, NS, 512)).astype(np.float32)
    lp = (rng.standard_normal((R, NS)) * 3).astype(np.float32)
    lp[3, 2] = -np.inf
    lp[5, :] = -np.inf
    lp[7, :8] = -np.inf
    lp[9, NS - 1] = -np.inf
    op[3, 2] = np.nan   # a split with lse = -inf adds nothing, whatever its O holds
    op[5, :] = np.nan
    op[9, NS - 1] = np.nan
    top = torch.from_numpy(op).to(DEV)
    tlp = torch.from_numpy(lp).to(DEV)
    o, lse = mla.splitkv_combine(top, tlp)
    torch.cuda.synchronize()
    ro, rl = oracle.combine(np.nan_to_num(op.astype(np.float64)), lp.astype(np.float64))
    check("host(lse)", host(lse), rl, 1e-5)
    # O is rounded to bf16 (round to nearest even): at most half a unit in the last place,
    # 2^-8 of |O| relative, plus the fp32 accumulation over <= 150 splits
    err = np.abs(host(o) - ro)
    bound = 2.0 ** -8 * np.abs(ro) + 1e-5
    say(f"  O: max |d| / bound = {float((err / bound).max()):.3f}")
    assert (err <= bound).all()
    assert (host(o)[5] == 0).all() and np.isneginf(host(lse)[5])


# ----------------------------------------------------------------------------------
# paged
# ----------------------------------------------------------------------------------

def _paged_run(w, num_splits=None, want_lse=True):
    d = paged_device_inputs(w)
    o, lse = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                              w.kv_scale, w.sm_scale, num_splits=num_splits, want_lse=want_lse)
    torch.cuda.synchronize()
    return host(o), (host(lse) if lse is not None else None)


def _paged_ref(w, requests=None):
    q, qpe = w.q_f64()
    return oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables,
                               w.seq_lens, w.sm_scale, requests=requests)


def _tol_o(fmt):
    return TOL_O_BF16 if fmt == gen.FMT_BF16 else TOL_O_QUANT


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4])
@pytest.mark.parametrize("q_len", [1, 2])
@pytest.mark.parametrize("page_size", [32, 64])
def test_paged_matches_oracle(fmt, q_len, page_size):
    say(f"paged fmt={gen.FMT_NAMES[fmt]} q_len={q_len} page={page_size}")
    w = gen.make_paged(B=4, H=128, q_len=q_len, lo=1, hi=400, page_size=page_size, fmt=fmt, seed=40 + fmt,
                       seq_lens=[1, 63, 290, 97], max_blocks=16, poison_tail=True)
    ro, rl = _paged_ref(w)
    for ns in (None, 1, 5):
        o, lse = _paged_run(w, ns)
        check_o(f"o {ns}", o, ro, _tol_o(fmt))
        check(f"lse {ns}", lse, rl, TOL_LSE)


@pytest.mark.parametrize("H,q_len", [(16, 1), (16, 2), (48, 1), (64, 4), (128, 8)])
def test_paged_head_and_query_counts(H, q_len):
    say(f"paged H={H} q_len={q_len}")
    w = gen.make_paged(B=3, H=H, q_len=q_len, lo=8, hi=200, page_size=64, fmt=gen.FMT_FP8, seed=50 + H + q_len,
                       max_blocks=4)
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


@pytest.mark.parametrize("ns", [None, 200])
def test_paged_one_long_request_spans_every_range(ns):
    """One 16000-token request beside a short one: the long request's rows merge one partial
    per range (up to 256, several rounds of 64 in the combine)."""
    say(f"paged one long request ns={ns}")
    w = gen.make_paged(B=2, H=16, q_len=1, lo=1, hi=1, page_size=64, fmt=gen.FMT_FP8, seed=63,
                       seq_lens=[16000, 40], max_blocks=250)
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w, ns)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_empty_and_short_requests():
    say("paged empty/short requests")
    w = gen.make_paged(B=5, H=32, q_len=2, lo=1, hi=1, page_size=32, fmt=gen.FMT_BF16, seed=60,
                       seq_lens=[0, 1, 2, 0, 33], max_blocks=3)
    ro, rl = _paged_ref(w)
    for ns in (None, 1, 2, 3):
        o, lse = _paged_run(w, ns)
        check_o(f"o {ns}", o, ro, TOL_O_BF16)
        check(f"lse {ns}", lse, rl, TOL_LSE)
        assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
        assert np.isneginf(lse[1, 0]).all() and (o[1, 0] == 0).all()


def test_paged_page_permutation_is_bitwise_invariant():
    say("paged page permutation")
    w = gen.make_paged(B=3, H=128, q_len=1, lo=100, hi=700, page_size=64, fmt=gen.FMT_FP8, seed=61)
    o1, l1 = _paged_run(w)
    rng = np.random.default_rng(1)
    perm = rng.permutation(w.num_pages)
    pages = w.cache.reshape(w.num_pages, w.page_stride)
    moved = np.empty_like(pages)
    moved[perm] = pages
    w.cache = moved.reshape(-1)
    w.block_tables = perm[w.block_tables].astype(np.int32)
    o2, l2 = _paged_run(w)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_padded_page_stride():
    say("paged padded stride")
    w = gen.make_paged(B=2, H=32, q_len=1, lo=50, hi=300, page_size=64, fmt=gen.FMT_NVFP4, seed=62,
                       page_stride=64 * 324 + 48)
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4])
def test_paged_pages_past_4gib(fmt):
    """A 4.6 GiB page pool whose used pages sit between 2 and 4 GiB and past 4 GiB into it:
    page byte offsets beyond the int32 and uint32 ranges (the oracle reads the same pages
    from a compact copy)."""
    say(f"paged pages past 4 GiB fmt={gen.FMT_NAMES[fmt]}")
    w = gen.make_paged(B=3, H=32, q_len=2, lo=1, hi=1, page_size=64, fmt=fmt, seed=64 + fmt,
                       seq_lens=[700, 2, 1500], poison_tail=True)
    ro, rl = _paged_ref(w)
    stride = w.page_stride
    big = int(4.6 * 2 ** 30) // stride
    lo2, lo4 = -(-2 ** 31 // stride), -(-2 ** 32 // stride)
    rng = np.random.default_rng(7)
    n = w.num_pages
    idx = np.concatenate([rng.choice(np.arange(lo2, lo4 - 1), n // 2, replace=False),
                          rng.choice(np.arange(lo4, big), n - n // 2, replace=False)]).astype(np.int64)
    rng.shuffle(idx)
    assert idx.min() * stride >= 2 ** 31 and (idx >= lo4).sum() == n - n // 2
    pool = torch.empty(big * stride, dtype=torch.uint8, device=DEV)
    pool.view(big, stride)[torch.from_numpy(idx).to(DEV)] = u8_dev(w.cache).view(n, stride)
    bt = i32_dev(idx[w.block_tables].astype(np.int32))
    d = paged_device_inputs(w)
    for ns in (None, 1):
        o, lse = mla.paged_decode(d["q"], d["qpe"], pool, w.fmt, bt, d["sl"], w.page_size, stride, w.kv_scale,
                                  w.sm_scale, num_splits=ns)
        torch.cuda.synchronize()
        check_o(f"o {ns}", host(o), ro, _tol_o(fmt))
        check(f"lse {ns}", host(lse), rl, TOL_LSE)
    del pool
    torch.cuda.empty_cache()


def test_paged_fp8_every_code():
    """A cache holding every E4M3 code (NaN codes excluded) decodes as the oracle does."""
    say("paged fp8 every code")
    w = gen.make_paged(B=1, H=16, q_len=1, lo=64, hi=64, page_size=64, fmt=gen.FMT_FP8, seed=63)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows = np.resize(codes, 64 * 576).reshape(64, 576)
    w.cache[:64 * 576] = rows.ravel()
    w.block_tables[:] = 0
    w.kv_scale = 1.0 / 128  # |values| <= 3.5 keeps the bf16 rounding of O inside the tolerance
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_nvfp4_every_code_and_scale():
    say("paged nvfp4 every code")
    w = gen.make_paged(B=1, H=16, q_len=1, lo=64, hi=64, page_size=64, fmt=gen.FMT_NVFP4, seed=64)
    rng = np.random.default_rng(2)
    page = w.cache[:64 * 324]
    page[:64 * 288] = np.resize(np.arange(256, dtype=np.uint8), 64 * 288)
    # scales up to 0.5 (codes 0x00..0x30 with either sign) keep |values| <= 3
    sc = np.array([c for c in range(256) if (c & 0x7F) <= 0x30], dtype=np.uint8)
    page[64 * 288:] = rng.choice(sc, 64 * 36)
    w.block_tables[:] = 0
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_nvfp4_large_scales():
    """Every E2M1 code under scales drawn from every finite E4M3 code of either sign, up to
    448 (values up to 2688, the top of the NVFP4 range, dequantised exactly to f16), with a
    query scaled by 2^-8 so that the scores stay moderate."""
    say("paged nvfp4 large scales")
    w = gen.make_paged(B=2, H=32, q_len=1, lo=300, hi=300, page_size=64, fmt=gen.FMT_NVFP4, seed=66)
    rng = np.random.default_rng(3)
    pages = w.cache.reshape(w.num_pages, w.page_stride)
    sc = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)  # no NaN codes
    for pg in range(w.num_pages - 1):  # the last page is the poison page
        pages[pg, :64 * 288] = rng.integers(0, 256, 64 * 288, dtype=np.uint8)
        pages[pg, 64 * 288:64 * 324] = rng.choice(sc, 64 * 36)
    w.q = _scale_bf16(w.q, -8)
    w.qpe = _scale_bf16(w.qpe, -8)
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    # O's error scales with the latent values: compare in units of the largest one
    vmax = max(float(np.abs(oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                                  w.block_tables[b], int(w.seq_lens[b]))[:, :512]).max())
               for b in range(w.B))
    say(f"  largest latent value {vmax:g}")
    assert vmax > 1000
    check_o("o / max|latent|", o / vmax, ro / vmax, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_fp8_b64_h128_full_size():
    """The benchmark workload at full size and in its benchmark launch configuration:
    every one of its 64 requests against the oracle."""
    say("paged_fp8_b64_h128 full size, all 64 requests")
    w = gen.make_workload("paged_fp8_b64_h128_s1k_32k")
    o, lse = _paged_run(w, mla.plan_paged(256, w.B, w.q_len, w.H))
    assert np.isfinite(o).all()
    ro, rl = _paged_ref(w)
    check_o("O (64 requests)", o, ro, TOL_O_QUANT)
    check("LSE (64 requests)", lse, rl, TOL_LSE)


def _scale_bf16(bits, k):
    """bf16 bits times 2^k (exact for these magnitudes)."""
    return gen.to_bf16_bits(gen.bf16_bits_to_f32(bits) * np.float32(2.0 ** k))


@pytest.mark.parametrize("fmt", [gen.FMT_FP8, gen.FMT_NVFP4, gen.FMT_BF16])
@pytest.mark.parametrize("qexp,scale_exp", [(12, -12), (-24, 24), (110, -110), (2, 0), (0, 0)])
def test_paged_query_magnitudes_and_peaked_rows(fmt, qexp, scale_exp):
    """The FP8 cache path splits each query row into two E4M3 operands after a power-of-two
    row scale, and the softmax weights likewise; the NVFP4 path scales each query row by a
    power of two into f16: query rows far from unit magnitude (the score scale compensates,
    so the scores are unchanged; 2^110 is near the top of the bf16 range), all-zero rows,
    and strongly peaked rows (query x 4: most weights fall below E4M3's subnormal range)
    stay within the tolerance of the oracle, as they do on the bf16 cache."""
    say(f"paged {gen.FMT_NAMES[fmt]} query x 2^{qexp}, sm_scale x 2^{scale_exp}")
    w = gen.make_paged(B=3, H=128, q_len=1, lo=200, hi=900, page_size=64, fmt=fmt, seed=65)
    w.q = _scale_bf16(w.q, qexp)
    w.qpe = _scale_bf16(w.qpe, qexp)
    w.q[:, :, :16] = 0
    w.qpe[:, :, :16] = 0
    w.sm_scale = w.sm_scale * 2.0 ** scale_exp
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, _tol_o(fmt))
    check("lse", lse, rl, TOL_LSE)


@pytest.mark.parametrize("q_len,page_size", [(1, 64), (2, 32)])
def test_paged_fp8_rising_scores(q_len, page_size):
    """Scores that rise along the sequence (positive queries, cache rows drifting along a
    positive direction) move the softmax reference many times, so the accumulators are
    rescaled on many tiles; the result still matches the oracle.  Also run with a single
    range, so that one workgroup walks both requests."""
    say(f"paged fp8 rising scores q_len={q_len} page={page_size}")
    w = gen.make_paged(B=2, H=128, q_len=q_len, lo=2000, hi=2000, page_size=page_size, fmt=gen.FMT_FP8, seed=66)
    rng = np.random.default_rng(4)
    w.q = gen.to_bf16_bits(np.abs(gen.bf16_bits_to_f32(w.q)))
    w.qpe = gen.to_bf16_bits(np.abs(gen.bf16_bits_to_f32(w.qpe)))
    pages = w.cache.reshape(w.num_pages, w.page_stride)
    rows = {}
    for b in range(w.B):
        n = int(w.seq_lens[b])
        npg = (n + page_size - 1) // page_size
        t = np.arange(npg * page_size, dtype=np.float32)
        # the score of token t grows by about 28 (natural units) over the request
        rows[b] = rng.standard_normal((npg * page_size, 576), dtype=np.float32) + (t / n)[:, None] * np.float32(0.85)
    w.kv_scale = float(np.float32(max(float(np.abs(r).max()) for r in rows.values())) / np.float32(448.0))
    for b in range(w.B):
        npg = rows[b].shape[0] // page_size
        pages[w.block_tables[b, :npg]] = gen.encode_pages(rows[b], w.fmt, page_size, w.page_stride, w.kv_scale)
    ro, rl = _paged_ref(w)
    for ns in (None, 1):
        o, lse = _paged_run(w, ns)
        check_o(f"o {ns}", o, ro, TOL_O_QUANT)
        check(f"lse {ns}", lse, rl, TOL_LSE)


@pytest.mark.parametrize("fmt", [gen.FMT_FP8, oracle.FMT_FP8_QFP8])
@pytest.mark.parametrize("where", ["first", "middle"])
def test_paged_fp8_dominant_token_over_long_tail(fmt, where):
    """One token scores 6-15 (natural units, by head) above a flat bulk of 32768 and 20000
    latent rows of mean 1, so that each bulk weight is 2^-9 .. 2^-21 of the dominant
    one while the bulk's total weight still rivals it.  The FP8 paths carry each
    tile's weights with their own power-of-two scale, so the bulk keeps its weight in
    both the numerator and the denominator; losing it in either shifts O by up to 1."""
    say(f"paged fp8 dominant token ({where}) over a long tail, fmt={fmt}")
    w = gen.make_paged(B=2, H=128, q_len=1, lo=1, hi=1, page_size=64, fmt=gen.FMT_FP8, seed=67,
                       seq_lens=[32768, 20000])
    rng = np.random.default_rng(11)
    pages = w.cache.reshape(w.num_pages, w.page_stride)
    rows, star = {}, {}
    for b in range(w.B):
        n = int(w.seq_lens[b])
        u = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=576)
        r = rng.standard_normal((gen.cdiv(n, 64) * 64, 576), dtype=np.float32) + np.float32(1.0)
        t = 0 if where == "first" else n // 2 + 17
        r[t] = u
        rows[b], star[b] = r, u
    w.kv_scale = float(np.float32(max(float(np.abs(r).max()) for r in rows.values())) / np.float32(448.0))
    for b in range(w.B):
        npg = rows[b].shape[0] // 64
        pages[w.block_tables[b, :npg]] = gen.encode_pages(rows[b], gen.FMT_FP8, 64, w.page_stride, w.kv_scale)
    alpha = np.linspace(0.14, 0.35, w.H, dtype=np.float32)  # per head
    q = np.empty((w.B, 1, w.H, 576), dtype=np.float32)
    for b in range(w.B):
        q[b, 0] = alpha[:, None] * star[b][None, :]
    w.q = gen.to_bf16_bits(q[..., :512])
    w.qpe = gen.to_bf16_bits(q[..., 512:])
    w.fmt = fmt
    ro, rl = _paged_ref(w)
    # the bulk carries a large share of the weight in most heads
    for ns in (None, 1):
        o, lse = _paged_run(w, ns)
        check_o(f"O ns={ns}", o, ro, TOL_O_QUANT)
        check(f"LSE ns={ns}", lse, rl, TOL_LSE)


# ----------------------------------------------------------------------------------
# sliding window and attention sinks (mla_paged_decode_ext)
# ----------------------------------------------------------------------------------

def _paged_run_ext(w, window, sinks, num_splits=None):
    d = paged_device_inputs(w)
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, dtype=np.float32)).to(DEV)
    o, lse = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                              w.kv_scale, w.sm_scale, num_splits=num_splits, window=window, sinks=sk)
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4, oracle.FMT_FP8_QFP8])
@pytest.mark.parametrize("q_len", [1, 3])
def test_paged_window_and_sinks_match_oracle(fmt, q_len):
    say(f"paged window+sinks fmt={fmt} q_len={q_len}")
    base_fmt = gen.FMT_FP8 if fmt == oracle.FMT_FP8_QFP8 else fmt
    w = gen.make_paged(B=4, H=64, q_len=q_len, lo=1, hi=400, page_size=32, fmt=base_fmt, seed=170 + fmt + q_len,
                       seq_lens=[1, 63, 290, 97], max_blocks=16, poison_tail=True)
    w.fmt = fmt
    q, qpe = w.q_f64()
    sinks = (np.random.default_rng(fmt + q_len).standard_normal(w.H) * 2).astype(np.float32)
    for window, sk in ((1, None), (2, sinks), (33, sinks), (100, None), (1000, sinks), (0, sinks)):
        ro, rl = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                     w.block_tables, w.seq_lens, w.sm_scale, window=window,
                                     sinks=None if sk is None else sk.astype(np.float64))
        for ns in (None, 1, 7):
            o, lse = _paged_run_ext(w, window, sk, ns)
            check_o(f"o {(window, ns)}", o, ro, _tol_o(base_fmt))
            check(f"lse {(window, ns)}", lse, rl, TOL_LSE)


def test_paged_ext_without_window_or_sinks_is_the_plain_path():
    w = gen.make_paged(B=3, H=32, q_len=2, lo=10, hi=300, page_size=64, fmt=gen.FMT_FP8, seed=181, max_blocks=5)
    o1, l1 = _paged_run(w)
    d = paged_device_inputs(w)
    call = mla.PagedCall(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                         w.kv_scale, w.sm_scale, window=0, sinks=None)
    o2, l2 = call.run()
    torch.cuda.synchronize()
    assert np.array_equal(o1, host(o2)) and np.array_equal(l1, host(l2))
    # window 1: every query sees its own token only, so O is that token's latent row (bf16)
    o3, _ = _paged_run_ext(w, 1, None)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        kv = oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables[b], n)
        for i in range(w.q_len):
            pos = n - w.q_len + i
            assert np.max(np.abs(o3[b, i] - kv[pos, :512][None, :])) <= TOL_O_QUANT


# ----------------------------------------------------------------------------------
# FP8 query (format 3): same FP8 pages, query rounded to E4M3, scores on FP8 MFMA
# ----------------------------------------------------------------------------------

def _fp8q(w):
    w.fmt = oracle.FMT_FP8_QFP8  # the FP8 workload's pages are the format's pages
    return w


@pytest.mark.parametrize("q_len", [1, 2])
@pytest.mark.parametrize("page_size", [32, 64])
def test_paged_fp8_query_matches_oracle(q_len, page_size):
    say(f"paged fp8-query q_len={q_len} page={page_size}")
    w = _fp8q(gen.make_paged(B=4, H=128, q_len=q_len, lo=1, hi=400, page_size=page_size, fmt=gen.FMT_FP8,
                             seed=140 + q_len + page_size, seq_lens=[1, 63, 290, 97], max_blocks=16,
                             poison_tail=True))
    ro, rl = _paged_ref(w)
    for ns in (None, 1, 5):
        o, lse = _paged_run(w, ns)
        check_o(f"o {ns}", o, ro, TOL_O_QUANT)
        check(f"lse {ns}", lse, rl, TOL_LSE)
    # the query really is rounded: the bf16-query path on the same pages differs
    w.fmt = gen.FMT_FP8
    o1, _ = _paged_run(w)
    assert max_err(o1, o) > 1e-3


@pytest.mark.parametrize("H,q_len", [(16, 1), (48, 2), (64, 4), (128, 8)])
def test_paged_fp8_query_head_and_query_counts(H, q_len):
    say(f"paged fp8-query H={H} q_len={q_len}")
    w = _fp8q(gen.make_paged(B=3, H=H, q_len=q_len, lo=8, hi=200, page_size=64, fmt=gen.FMT_FP8,
                             seed=150 + H + q_len, max_blocks=4))
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_fp8_query_rounding_ties_and_every_code():
    """Every E4M3 code in the cache, and a query made of exact E4M3 midpoints (as bf16), so
    the kernel's rounding of the query must break every tie as the oracle does."""
    say("paged fp8-query ties")
    w = _fp8q(gen.make_paged(B=1, H=16, q_len=1, lo=64, hi=64, page_size=64, fmt=gen.FMT_FP8, seed=163))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    w.cache[:64 * 576] = np.resize(codes, 64 * 576)
    w.block_tables[:] = 0
    w.kv_scale = 1.0 / 128
    v = oracle.decode_e4m3fn(np.arange(0x7F))
    mids = ((v[:-1] + v[1:]) / 2)
    mids = mids[(mids > 0.1) & (mids < 3)]  # keep the scores moderate
    rng = np.random.default_rng(7)
    vals = rng.choice(mids, size=w.q.size + w.qpe.size) * rng.choice([-1.0, 1.0], size=w.q.size + w.qpe.size)
    bits = gen.to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(gen.bf16_bits_to_f32(bits), vals.astype(np.float32))  # exact in bf16
    w.q = bits[:w.q.size].reshape(w.q.shape)
    w.qpe = bits[w.q.size:].reshape(w.qpe.shape)
    ro, rl = _paged_ref(w)
    o, lse = _paged_run(w)
    check_o("o", o, ro, TOL_O_QUANT)
    check("lse", lse, rl, TOL_LSE)


def test_paged_fp8_query_b64_h128_full_size_sampled():
    """The FP8-query format on the benchmark pages: 16 requests (every fourth, sorted by
    length, so the shortest and the longest are among them)."""
    say("paged_fp8_b64_h128 fp8-query full size, 16 requests")
    w = _fp8q(gen.make_workload("paged_fp8_b64_h128_s1k_32k"))
    o, lse = _paged_run(w, mla.plan_paged(256, w.B, w.q_len, w.H))
    assert np.isfinite(o).all()
    order = np.argsort(w.seq_lens)
    pick = sorted({int(order[i]) for i in list(range(0, 64, 4)) + [63]})
    ro, rl = _paged_ref(w, requests=pick)
    check_o(f"O ({len(pick)} requests)", o[pick], ro, TOL_O_QUANT)
    check(f"LSE ({len(pick)} requests)", lse[pick], rl, TOL_LSE)


@pytest.mark.slow
def test_paged_nvfp4_b128_h128_q2_full_size_sampled():
    """The NVFP4 q_len 2 workload at full size and in its benchmark launch configuration:
    16 of its 128 requests (every eighth by length, with the shortest and the longest)."""
    say("paged_nvfp4_b128_h128_q2 full size, 16 requests")
    w = gen.make_workload("paged_nvfp4_b128_h128_q2_s2k_64k")
    o, lse = _paged_run(w, mla.plan_paged(256, w.B, w.q_len, w.H))
    assert np.isfinite(o).all()
    order = np.argsort(w.seq_lens)
    pick = sorted({int(order[i]) for i in list(range(0, 128, 8)) + [127]})
    ro, rl = _paged_ref(w, requests=pick)
    check_o(f"O ({len(pick)} requests)", o[pick], ro, TOL_O_QUANT)
    check(f"LSE ({len(pick)} requests)", lse[pick], rl, TOL_LSE)


@pytest.mark.parametrize("fmt", [gen.FMT_BF16, gen.FMT_FP8])
def test_paged_batch_with_no_tokens(fmt):
    """Every request empty (the decode finds no tiles at all and stops after its plan): O
    is zero and LSE -inf for every row, through all three paged entry points, with sinks
    the LSE is the sink."""
    say(f"paged all-empty batch fmt={fmt}")
    w = gen.make_paged(B=3, H=16, q_len=2, lo=0, hi=0, page_size=64, fmt=fmt, seed=70, seq_lens=[0, 0, 0],
                       max_blocks=2)
    d = paged_device_inputs(w)
    o, lse = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                              w.kv_scale, w.sm_scale)
    o2, lse2, _, _ = mla.paged_decode_splits(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size,
                                             w.page_stride, w.kv_scale, w.sm_scale)
    sinks = torch.linspace(-1.0, 1.0, w.H, device=DEV)
    o3, lse3 = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                                w.kv_scale, w.sm_scale, sinks=sinks)
    torch.cuda.synchronize()
    for oo, ll in ((o, lse), (o2, lse2)):
        assert (host(oo) == 0).all() and np.isneginf(host(ll)).all()
    assert (host(o3) == 0).all()
    assert np.array_equal(host(lse3), np.broadcast_to(host(sinks), (3, 2, w.H)))


@pytest.mark.parametrize("fmt,sinks", [(gen.FMT_FP8, False), (gen.FMT_BF16, True)])
def test_paged_single_long_request_over_every_range(fmt, sinks):
    """One 32768-token request over all the device's ranges (256 partials per row): the
    combine takes a workgroup per row for requests this wide; with sinks as well."""
    say(f"paged single long request fmt={fmt} sinks={sinks}")
    w = gen.make_paged(B=1, H=128, q_len=1, lo=32768, hi=32768, page_size=64, fmt=fmt, seed=90 + fmt)
    d = paged_device_inputs(w)
    sk = torch.linspace(-2.0, 6.0, w.H, device=DEV) if sinks else None
    o, lse = mla.paged_decode(d["q"], d["qpe"], d["cache"], w.fmt, d["bt"], d["sl"], w.page_size, w.page_stride,
                              w.kv_scale, w.sm_scale, num_splits=mla.plan_paged(256, w.B, w.q_len, w.H), sinks=sk)
    torch.cuda.synchronize()
    q, qpe = w.q_f64()
    ro, rl = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables,
                                 w.seq_lens, w.sm_scale,
                                 sinks=None if sk is None else host(sk).astype(np.float64))
    check_o("O", host(o), ro, _tol_o(fmt))
    check("LSE", host(lse), rl, TOL_LSE)
