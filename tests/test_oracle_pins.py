"""Pins of the float64 oracle to things other than itself (CPU only).

Each test checks the oracle against what the pages and the mathematics fix: brute
force on tiny inputs, torch's float64 SDPA (an independent implementation of the same
definition), closed forms, invariances, torch's own float8 decode, the OCP MX E2M1
table and quantisation error bounds.  ``test_pins_catch_planted_mistakes`` plants
plausible mistakes in copies of the oracle's attention and checks that a pin fails.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))
    assert np.nanmax(ours) == 448.0


def test_e2m1_matches_ocp_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) if ln[0] != "#"]
    table = {int(a): float(b) for a, b in rows}
    ours = oracle.decode_e2m1(np.arange(16))
    for c in range(16):
        assert ours[c] == table[c], c
        assert np.signbit(ours[c]) == np.signbit(table[c]), c


def test_bf16_bits_decode_matches_torch():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_nvfp4_products_exact_in_bf16():
    """Every E2M1 value times every finite E4M3 scale is exactly a bf16 value, so a
    bf16 tile holds the dequantised NVFP4 cache without rounding."""
    v = oracle.decode_e2m1(np.arange(16))
    s = oracle.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    s = s[np.isfinite(s)]
    prod = (v[:, None] * s[None, :]).ravel()
    back = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, prod)


def test_fp8_values_exact_in_bf16():
    s = oracle.decode_e4m3fn(np.arange(256, dtype=np.uint8))
    s = s[np.isfinite(s)]
    back = torch.from_numpy(s).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, s)


def test_fp8_page_decode_within_quantisation_bound():
    rng = np.random.default_rng(11)
    P = 32
    x = rng.standard_normal((P, oracle.ROW), dtype=np.float32)
    scale = float(np.float32(np.abs(x).max()) / np.float32(448))
    page = gen.encode_pages(x, gen.FMT_FP8, P, P * oracle.ROW, scale)[0]
    dec = oracle.decode_page(page, oracle.FMT_FP8, P, scale)
    # E4M3: relative half-ulp 2^-4 for normals, absolute 2^-10 below 2^-6
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale)
    assert (np.abs(dec - x) <= bound * 1.0000001 + 1e-12).all()
    # codes come from torch's cast, so the decode must equal torch's decode exactly
    ref = torch.from_numpy(page[:P * oracle.ROW].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(dec.ravel(), scale * ref)


def test_nvfp4_page_decode_within_quantisation_bound():
    """The generator's encoder writes the reading of the NVFP4 page independently of the
    oracle's decoder; a wrong nibble order, group or section offset in either breaks the
    E2M1 error bound |x - deq| <= s_g (largest grid gap 2, times half, plus saturation)."""
    rng = np.random.default_rng(12)
    P = 16
    x = rng.standard_normal((P, oracle.ROW), dtype=np.float32)
    stride = P * (oracle.ROW // 2 + oracle.ROW // 16)
    page = gen.encode_pages(x, gen.FMT_NVFP4, P, stride, 1.0)[0]
    dec = oracle.decode_page(page, oracle.FMT_NVFP4, P)
    sc = oracle.decode_e4m3fn(page[P * 288:P * 324].reshape(P, 36))
    bound = np.repeat(sc, 16, axis=1)
    assert (np.abs(dec - x) <= bound + 1e-12).all()
    # and the decode is far better than the bound on average
    assert np.mean(np.abs(dec - x) / bound) < 0.3


# ----------------------------------------------------------------------------------
# attention: brute force, library routine, closed forms
# ----------------------------------------------------------------------------------

def brute_force_attend(qfull, kv, visible, sm_scale):
    """Pure-Python loops over the definition (no numpy reductions)."""
    R, n = len(qfull), len(kv)
    O = [[0.0] * 512 for _ in range(R)]
    L = [-math.inf] * R
    for r in range(R):
        v = min(max(int(visible[r]), 0), n)
        if v == 0:
            continue
        s = []
        for t in range(v):
            acc = 0.0
            for d in range(576):
                acc += float(qfull[r][d]) * float(kv[t][d])
            s.append(sm_scale * acc)
        m = max(s)
        z = sum(math.exp(x - m) for x in s)
        L[r] = m + math.log(z)
        for t in range(v):
            w = math.exp(s[t] - L[r])
            for d in range(512):
                O[r][d] += w * float(kv[t][d])
    return np.array(O), np.array(L)


def test_attend_matches_brute_force():
    rng = np.random.default_rng(1)
    qf = _rand(rng, 3, 576)
    kv = _rand(rng, 23, 576)
    vis = np.array([23, 7, 1])
    O, L = oracle.attend(qf, kv, vis, 0.07)
    Ob, Lb = brute_force_attend(qf, kv, vis, 0.07)
    assert np.abs(O - Ob).max() < 1e-12
    assert np.abs(L - Lb).max() < 1e-12


def sdpa_reference(qfull, kv, visible, sm_scale):
    q = torch.from_numpy(qfull)[None, None]           # [1,1,R,576]
    k = torch.from_numpy(kv)[None, None]              # [1,1,n,576]
    v = torch.from_numpy(kv[:, :512].copy())[None, None]
    mask = torch.arange(kv.shape[0])[None, :] < torch.from_numpy(np.asarray(visible))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=sm_scale)
    scores = (q @ k.transpose(-1, -2))[0, 0] * sm_scale
    lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
    return o[0, 0].numpy(), lse.numpy()


def _attend_vs_sdpa(attend_fn, seed=2):
    rng = np.random.default_rng(seed)
    qf = _rand(rng, 8, 576)
    kv = _rand(rng, 300, 576)
    vis = np.array([300, 299, 150, 1, 64, 65, 2, 300])
    O, L = attend_fn(qf, kv, vis, 1.0 / math.sqrt(192))
    Or, Lr = sdpa_reference(qf, kv, vis, 1.0 / math.sqrt(192))
    return max(np.abs(O - Or).max(), np.abs(L - Lr).max())


def test_attend_matches_torch_sdpa_float64():
    assert _attend_vs_sdpa(oracle.attend) < 1e-10


def test_closed_form_zero_query_is_mean():
    rng = np.random.default_rng(3)
    kv = _rand(rng, 100, 576)
    qf = np.zeros((2, 576))
    O, L = oracle.attend(qf, kv, np.array([100, 37]), 0.1)
    assert np.abs(O[0] - kv[:100, :512].mean(0)).max() < 1e-13
    assert np.abs(O[1] - kv[:37, :512].mean(0)).max() < 1e-13
    assert abs(L[0] - math.log(100)) < 1e-13 and abs(L[1] - math.log(37)) < 1e-13
    # sm_scale = 0 gives the same with any query
    O2, L2 = oracle.attend(_rand(rng, 2, 576), kv, np.array([100, 37]), 0.0)
    assert np.abs(O2 - O).max() < 1e-13 and np.abs(L2 - L).max() < 1e-13


def test_closed_form_single_token_and_dominant_token():
    rng = np.random.default_rng(4)
    kv = _rand(rng, 50, 576)
    qf = _rand(rng, 1, 576)
    O, L = oracle.attend(qf, kv, np.array([1]), 0.3)
    assert np.array_equal(O[0], kv[0, :512])
    assert abs(L[0] - 0.3 * float(qf[0] @ kv[0])) < 1e-12
    tstar = 17
    qd = (40.0 * kv[tstar])[None]
    Od, _ = oracle.attend(qd, kv, np.array([50]), 1.0)
    assert np.abs(Od[0] - kv[tstar, :512]).max() < 1e-9


def test_empty_rows():
    kv = np.ones((5, 576))
    O, L = oracle.attend(np.ones((2, 576)), kv, np.array([0, -3]), 1.0)
    assert (O == 0).all() and np.isneginf(L).all()
    O, L = oracle.attend(np.ones((2, 576)), np.zeros((0, 576)), np.array([0, 0]), 1.0)
    assert (O == 0).all() and np.isneginf(L).all()


# ----------------------------------------------------------------------------------
# split-KV: invariance and merge identity
# ----------------------------------------------------------------------------------

def test_split_invariance_contig():
    rng = np.random.default_rng(6)
    B, H, S = 2, 4, 300
    q, qpe = _rand(rng, B, H, 512), _rand(rng, B, H, 64)
    kv, kpe = _rand(rng, B, S, 512), _rand(rng, B, S, 64)
    O, L = oracle.contig_decode(q, qpe, kv, kpe, 0.05)
    for Ls in (1, 7, 64, 128, S):
        op, lp = oracle.contig_decode_splitkv(q, qpe, kv, kpe, 0.05, Ls)
        assert op.shape == (B, H, oracle.cdiv(S, Ls), 512)
        Oc, Lc = oracle.combine(op.reshape(B * H, -1, 512), lp.reshape(B * H, -1))
        assert np.abs(Oc.reshape(B, H, 512) - O).max() < 1e-12, Ls
        assert np.abs(Lc.reshape(B, H) - L).max() < 1e-12, Ls


def test_lse_merge_identity():
    rng = np.random.default_rng(7)
    qf = _rand(rng, 3, 576)
    kv = _rand(rng, 90, 576)
    vis = np.full(3, 90)
    for a, b in ((0, 90), (13, 90), (0, 1), (45, 46)):
        oa, la = oracle.attend_range(qf, kv, vis, 0.2, 0, a)
        ob, lb = oracle.attend_range(qf, kv, vis, 0.2, a, b)
        oab, lab = oracle.attend_range(qf, kv, vis, 0.2, 0, b)
        Om, Lm = oracle.combine(np.stack([oa, ob], 1), np.stack([la, lb], 1))
        assert np.abs(Om - oab).max() < 1e-12 and np.abs(Lm - lab).max() < 1e-12
    # an empty part (lse = -inf, O = 0) is the identity
    o1, l1 = oracle.attend_range(qf, kv, vis, 0.2, 0, 90)
    Om, Lm = oracle.combine(np.stack([o1, np.zeros_like(o1)], 1), np.stack([l1, np.full(3, -np.inf)], 1))
    assert np.array_equal(Om, o1) and np.array_equal(Lm, l1)
    # all parts empty -> O = 0, LSE = -inf
    Oe, Le = oracle.combine(np.zeros((2, 3, 512)), np.full((2, 3), -np.inf))
    assert (Oe == 0).all() and np.isneginf(Le).all()


# ----------------------------------------------------------------------------------
# paged: gather, permutation invariance, causal verify
# ----------------------------------------------------------------------------------

def test_paged_equals_contig_on_same_rows():
    """A bf16 page pool holding the contiguous rows in a shuffled page order gives the
    same result as the contiguous op: pins the gather (page = table[t // P], row t % P)."""
    rng = np.random.default_rng(8)
    B, H, S, P = 2, 4, 200, 32
    c = gen.make_contig(B, H, S, seed=99)
    q, qpe, kv, kpe = c.f64()
    O, L = oracle.contig_decode(q, qpe, kv, kpe, 0.1)
    npg = oracle.cdiv(S, P)
    perm = rng.permutation(B * npg)
    stride = P * 1152
    cache = np.zeros((B * npg, stride), np.uint8)
    rows = np.concatenate([c.kv, c.kpe], axis=-1)  # bf16 bits [B,S,576]
    bt = np.zeros((B, npg), np.int32)
    for b in range(B):
        for i in range(npg):
            blk = np.zeros((P, 576), np.uint16)
            part = rows[b, i * P:(i + 1) * P]
            blk[:len(part)] = part
            cache[perm[b * npg + i]] = blk.view(np.uint8).ravel()
            bt[b, i] = perm[b * npg + i]
    Op, Lp = oracle.paged_decode(q[:, None], qpe[:, None], cache.ravel(), oracle.FMT_BF16, 1.0, P, stride, bt,
                                 np.full(B, S), 0.1)
    assert np.array_equal(Op[:, 0], O) and np.array_equal(Lp[:, 0], L)


def test_page_permutation_invariance():
    w = gen.make_paged(B=3, H=4, q_len=2, lo=70, hi=300, page_size=32, fmt=gen.FMT_FP8, seed=21)
    q, qpe = w.q_f64()
    O, L = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                               w.block_tables, w.seq_lens, w.sm_scale)
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.num_pages)
    pages = w.cache.reshape(w.num_pages, w.page_stride)
    moved = np.empty_like(pages)
    moved[perm] = pages
    bt2 = perm[w.block_tables]
    O2, L2 = oracle.paged_decode(q, qpe, moved.ravel(), w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                 bt2, w.seq_lens, w.sm_scale)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    assert np.isfinite(O).all()


def test_paged_split_partials_merge_to_the_whole_and_clip_at_the_length():
    """Fixed-length splits of the paged op: merging the partials gives the unsplit
    result; split j of a request equals attention over that request's tokens [jL, (j+1)L)
    alone (brute force on the gathered rows); splits at or past the length are empty."""
    w = gen.make_paged(B=4, H=3, q_len=2, lo=1, hi=1, page_size=32, fmt=gen.FMT_FP8, seed=23,
                       seq_lens=[0, 1, 130, 300], max_blocks=10)
    q, qpe = w.q_f64()
    args = (q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables, w.seq_lens, w.sm_scale)
    O, L = oracle.paged_decode(*args)
    for Ls, ns in ((128, 3), (128, 5), (256, 2), (512, 1)):
        op, lp = oracle.paged_decode_split_partials(*args, Ls, ns)
        assert op.shape == (4, 2, 3, ns, 512) and lp.shape == (4, 2, 3, ns)
        Oc, Lc = oracle.combine(op.reshape(-1, ns, 512), lp.reshape(-1, ns))
        assert np.abs(Oc.reshape(O.shape) - O).max() < 1e-12, Ls
        fin = np.isfinite(L)
        assert np.array_equal(np.isfinite(Lc.reshape(L.shape)), fin)
        assert np.abs(Lc.reshape(L.shape)[fin] - L[fin]).max() < 1e-12, Ls
        for b, n in enumerate(w.seq_lens):
            for j in range(ns):
                if j * Ls >= n:
                    assert np.isneginf(lp[b, :, :, j]).all() and (op[b, :, :, j] == 0).all()
    # the FP8-query format rounds the query before splitting, as the unsplit op does
    qargs = (q, qpe, w.cache, oracle.FMT_FP8_QFP8) + args[4:]
    Oq, Lq = oracle.paged_decode(*qargs)
    op, lp = oracle.paged_decode_split_partials(*qargs, 128, 3)
    Oc, _ = oracle.combine(op.reshape(-1, 3, 512), lp.reshape(-1, 3))
    assert np.abs(Oc.reshape(Oq.shape) - Oq).max() < 1e-12 and np.abs(Oq - O).max() > 1e-6
    # brute force: request 3 (300 tokens), split 1 of L = 128 covers tokens 128..255; query 0
    # sees 299 tokens, so all of them; one head
    kv = oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables[3], 300)
    op, lp = oracle.paged_decode_split_partials(*args, 128, 3)
    qf = np.concatenate([q[3, 0, 1], qpe[3, 0, 1]])
    s = np.array([w.sm_scale * float(qf @ kv[t]) for t in range(128, 256)])
    p = np.exp(s - s.max())
    assert abs(lp[3, 0, 1, 1] - (s.max() + math.log(p.sum()))) < 1e-12
    assert np.abs(op[3, 0, 1, 1] - (p / p.sum()) @ kv[128:256, :512]).max() < 1e-12
    # request 3, split 2 (256..299): query 0 sees tokens up to 298 -> 43 tokens, query 1 all 44
    s0 = np.array([w.sm_scale * float(np.concatenate([q[3, 0, 0], qpe[3, 0, 0]]) @ kv[t]) for t in range(256, 299)])
    assert abs(lp[3, 0, 0, 2] - (s0.max() + math.log(np.exp(s0 - s0.max()).sum()))) < 1e-12
    # request 1 (one token): query 0 sees nothing, query 1 sees token 0 with weight 1
    assert np.isneginf(lp[1, 0]).all() and (op[1, 0] == 0).all()
    kv1 = oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables[1], 1)
    assert np.abs(op[1, 1, :, 0] - kv1[0, :512]).max() < 1e-12


def test_causal_verify_rows():
    """q_len = 2: query 0 sees n-1 tokens and equals a one-token decode over n-1 tokens;
    query 1 sees all n; zero queries give ln(n-1) and ln(n)."""
    w = gen.make_paged(B=2, H=4, q_len=2, lo=65, hi=130, page_size=64, fmt=gen.FMT_BF16, seed=22)
    q, qpe = w.q_f64()
    O, L = oracle.paged_decode(q, qpe, w.cache, w.fmt, 1.0, w.page_size, w.page_stride,
                               w.block_tables, w.seq_lens, w.sm_scale)
    for b in range(2):
        n = int(w.seq_lens[b])
        o0, l0 = oracle.paged_decode_request(q[b, :1], qpe[b, :1], w.cache, w.fmt, 1.0, w.page_size,
                                             w.page_stride, w.block_tables[b], n - 1, w.sm_scale)
        assert np.array_equal(o0[0], O[b, 0]) and np.array_equal(l0[0], L[b, 0])
    Oz, Lz = oracle.paged_decode(np.zeros_like(q), np.zeros_like(qpe), w.cache, w.fmt, 1.0, w.page_size,
                                 w.page_stride, w.block_tables, w.seq_lens, w.sm_scale)
    for b in range(2):
        n = int(w.seq_lens[b])
        assert np.abs(Lz[b, 0] - math.log(n - 1)).max() < 1e-12
        assert np.abs(Lz[b, 1] - math.log(n)).max() < 1e-12


def test_seq_len_below_q_len_gives_empty_row():
    w = gen.make_paged(B=2, H=2, q_len=2, lo=1, hi=1, page_size=32, fmt=gen.FMT_BF16, seed=23,
                       seq_lens=[1, 0])
    q, qpe = w.q_f64()
    O, L = oracle.paged_decode(q, qpe, w.cache, w.fmt, 1.0, w.page_size, w.page_stride,
                               w.block_tables, w.seq_lens, w.sm_scale)
    assert np.isneginf(L[0, 0]).all() and (O[0, 0] == 0).all()
    assert np.isfinite(L[0, 1]).all()
    assert np.isneginf(L[1]).all() and (O[1] == 0).all()


def test_poisoned_table_entries_are_never_read():
    w = gen.make_paged(B=3, H=2, q_len=1, lo=40, hi=200, page_size=32, fmt=gen.FMT_NVFP4, seed=24,
                       max_blocks=16, poison_tail=True)
    q, qpe = w.q_f64()
    O, L = oracle.paged_decode(q, qpe, w.cache, w.fmt, 1.0, w.page_size, w.page_stride,
                               w.block_tables, w.seq_lens, w.sm_scale)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    assert (w.block_tables == w.poison_page).any()


# ----------------------------------------------------------------------------------
# planner
# ----------------------------------------------------------------------------------

def test_next_power_of_2_definition():
    assert oracle.next_power_of_2(0) == 1 and oracle.next_power_of_2(-5) == 1
    for n in list(range(1, 5000)) + [2 ** 20 - 1, 2 ** 20, 2 ** 20 + 1]:
        assert oracle.next_power_of_2(n) == 2 ** math.ceil(math.log2(n)), n


def test_contig_planner_worked_examples():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "planner_tilegym.txt")) if ln[0] != "#"]
    for cus, B, S, L, NS in (map(int, r) for r in rows):
        assert oracle.plan_contig(cus, B, S) == (L, NS), (cus, B, S)


def test_contig_planner_invariants():
    for B in (1, 2, 3, 7, 64, 255, 256, 1000):
        for S in (1, 127, 128, 129, 4096, 8191, 100000):
            L, NS = oracle.plan_contig(256, B, S)
            assert L >= 128 and L & (L - 1) == 0
            assert (NS - 1) * L < S <= NS * L


# ----------------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------------

def _mutant(kind):
    def attend(qfull, kv, visible, sm_scale):
        qfull = np.asarray(qfull, np.float64)
        kv = np.asarray(kv, np.float64)
        R, n = qfull.shape[0], kv.shape[0]
        O = np.zeros((R, 512))
        lse = np.full(R, -np.inf)
        nope = qfull[:, :512] @ kv[:, :512].T
        rope = qfull[:, 512:] @ kv[:, 512:].T
        if kind == "drop_rope":
            s = sm_scale * nope
        elif kind == "rope_sign":
            s = sm_scale * (nope - rope)
        elif kind == "scale_sqrt":
            s = math.sqrt(sm_scale) * (nope + rope)
        else:
            s = sm_scale * (nope + rope)
        for r in range(R):
            v = int(min(max(visible[r], 0), n))
            if kind == "off_by_one_visible":
                v = max(v - 1, 0)
            if v == 0:
                continue
            sr = s[r, :v]
            m = sr.max()
            lse[r] = m + math.log(np.exp(sr - m).sum())
            vals = kv[:v, 64:576] if kind == "v_from_wrong_columns" else kv[:v, :512]
            O[r] = np.exp(sr - lse[r]) @ vals
            if kind == "lse_base2":
                lse[r] = lse[r] / math.log(2)
        return O, lse
    return attend


@pytest.mark.parametrize("kind", ["drop_rope", "rope_sign", "scale_sqrt", "off_by_one_visible",
                                  "v_from_wrong_columns", "lse_base2"])
def test_pins_catch_planted_mistakes(kind):
    assert _attend_vs_sdpa(_mutant("none")) < 1e-10
    assert _attend_vs_sdpa(_mutant(kind)) > 1e-3


# ----------------------------------------------------------------------------------
# cache append: the quantisers and the row placement
# ----------------------------------------------------------------------------------

def _e4m3_midpoints():
    """Every midpoint between adjacent non-negative finite E4M3 values (exact in fp32)."""
    v = oracle.decode_e4m3fn(np.arange(0x7F))
    return ((v[:-1] + v[1:]) / 2).astype(np.float32), np.arange(0x7E)


def test_e4m3_quantiser_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.decode_e4m3fn(codes).astype(np.float32)
    assert np.array_equal(oracle.quantize_e4m3(vals), codes)


def test_e4m3_quantiser_matches_torch_cast():
    # torch's float8_e4m3fn cast rounds to nearest, ties to even (no saturation, so the
    # inputs stay within +-448); random values, every midpoint, and its neighbours
    rng = np.random.default_rng(11)
    mids, _ = _e4m3_midpoints()
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(50),
                        rng.uniform(-2 ** -5, 2 ** -5, 5000).astype(np.float32),
                        mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500))])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.quantize_e4m3(x), ref)


def test_e4m3_quantiser_hand_cases():
    # ties go to the even code; saturation at 448; the sign of zero is kept
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2 ** -10, 0x00), (3 * 2 ** -10, 0x02), (1000.0, 0x7E),
             (-1000.0, 0xFE), (448.0, 0x7E), (464.0, 0x7E), (240.0, 0x77), (-0.0, 0x80), (-1e-6, 0x80),
             (0.0, 0x00), (2 ** -6, 0x08)]
    for x, c in cases:
        assert int(oracle.quantize_e4m3(np.float32(x))) == c, (x, c)


def test_e2m1_quantiser_cases():
    vals = oracle.decode_e2m1(np.arange(16)).astype(np.float32)
    assert np.array_equal(oracle.quantize_e2m1(vals), np.arange(16, dtype=np.uint8))
    # midpoints tie to the even code (0, 1, 2, 4 have even codes); saturation at 6
    cases = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (5.0001, 7), (7.0, 7),
             (1e9, 7), (-0.25, 8), (-5.0, 14), (-0.1, 8), (0.2500001, 1), (0.7499999, 1), (-0.0, 8), (0.0, 0)]
    for x, c in cases:
        assert int(oracle.quantize_e2m1(np.float32(x))) == c, (x, c)


def test_encode_row_matches_input_recipe_encoders():
    # the input recipe encodes with torch's cast and its own threshold table: an
    # implementation of the same readings that shares no code with the oracle
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, oracle.ROW)).astype(np.float32)
    bits = gen.to_bf16_bits(x)
    xb = gen.bf16_bits_to_f32(bits)
    s = np.float32(0.0173)
    fp8_ref = gen.to_e4m3_codes(xb / s)
    d_ref, sc_ref = gen.encode_nvfp4_rows(xb)
    for r in range(64):
        assert np.array_equal(oracle.encode_row(bits[r], oracle.FMT_FP8, float(s)), fp8_ref[r])
        enc = oracle.encode_row(bits[r], oracle.FMT_NVFP4)
        assert np.array_equal(enc[:288], d_ref[r])
        assert np.array_equal(enc[288:], sc_ref[r])
        assert np.array_equal(oracle.encode_row(bits[r], oracle.FMT_BF16).view(np.uint16), bits[r])


def test_encode_row_error_bounds():
    # FP8: |x - kv_scale * e4m3(code)| <= half a step of the E4M3 grid at |x / kv_scale|;
    # NVFP4: per group the scale is the E4M3 value nearest amax / 6, and each value is
    # within half an E2M1 step (times the scale) of its code's value
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((16, oracle.ROW)) * 3).astype(np.float32)
    bits = gen.to_bf16_bits(x)
    xb = gen.bf16_bits_to_f32(bits).astype(np.float64)
    s = 0.05
    for r in range(16):
        y = xb[r] / s
        got = oracle.decode_e4m3fn(oracle.encode_row(bits[r], oracle.FMT_FP8, s))
        ulp = np.where(np.abs(y) < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-30))) - 3))
        assert np.all(np.abs(got - y) <= ulp / 2 + 1e-12)
        enc = oracle.encode_row(bits[r], oracle.FMT_NVFP4)
        page = np.zeros(324, dtype=np.uint8)
        page[:324] = enc
        dec = oracle.decode_page(page, oracle.FMT_NVFP4, 1)[0]
        g = xb[r].reshape(36, 16)
        sc = oracle.decode_e4m3fn(enc[288:])
        for k in range(36):
            amax = np.abs(g[k]).max()
            cand = oracle.decode_e4m3fn(np.arange(0x7F))
            assert abs(sc[k] - amax / 6) <= np.min(np.abs(cand - amax / 6)) + 1e-12
            if sc[k] > 0:
                a = np.abs(g[k] / sc[k])
                step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
                err = np.abs(dec.reshape(36, 16)[k] / sc[k] - g[k] / sc[k])
                assert np.all(err <= np.maximum(step / 2, a - 6) + 1e-9)


def test_kv_append_places_rows_and_skips_outside_slots():
    rng = np.random.default_rng(14)
    page_size, num_pages = 32, 5
    for fmt in (oracle.FMT_BF16, oracle.FMT_FP8, oracle.FMT_NVFP4):
        stride = page_size * oracle.page_row_bytes(fmt) + 48
        cache = rng.integers(0, 256, num_pages * stride, dtype=np.uint8)
        lat = gen.to_bf16_bits(rng.standard_normal((4, 512)).astype(np.float32))
        rope = gen.to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32))
        slots = np.array([-1, 3 * page_size + 7, num_pages * page_size, 0])
        out = oracle.kv_append(cache, lat, rope, slots, fmt, 0.25, page_size, stride, num_pages)
        changed = np.nonzero(out != cache)[0]
        # only the rows of slots 3*32+7 and 0 (and their NVFP4 scales) may change
        rb = oracle.page_row_bytes(fmt) if fmt != oracle.FMT_NVFP4 else 288
        allowed = set(range(3 * stride + 7 * rb, 3 * stride + 8 * rb)) | set(range(0, rb))
        if fmt == oracle.FMT_NVFP4:
            allowed |= set(range(3 * stride + 32 * 288 + 7 * 36, 3 * stride + 32 * 288 + 8 * 36))
            allowed |= set(range(32 * 288, 32 * 288 + 36))
        assert set(changed.tolist()) <= allowed
        # reading back through decode_page gives the encoded row
        for j, slot in ((1, 3 * page_size + 7), (3, 0)):
            p, r = divmod(slot, page_size)
            dec = oracle.decode_page(out[p * stride:(p + 1) * stride], fmt, page_size, 0.25)[r]
            want = oracle.decode_bf16_bits(np.concatenate([lat[j], rope[j]]))
            if fmt == oracle.FMT_BF16:
                assert np.array_equal(dec, want)
            elif fmt == oracle.FMT_FP8:  # half an E4M3 step: 2^-4 relative, 2^-10 * scale near zero
                assert np.all(np.abs(dec - want) <= np.abs(want) * 2.0 ** -4 + 0.25 * 2.0 ** -10)
            else:  # half an E2M1 step of the group's scale (<= amax / 6 * 1.07)
                assert np.max(np.abs(dec - want)) < 1.5


@pytest.mark.parametrize("kind", ["ties_away", "truncate", "no_saturation"])
def test_quantiser_pins_catch_planted_mistakes(kind, monkeypatch):
    """Plant a plausible rounding mistake in a copy of the nearest-even search and check
    that the torch-cast and hand-case pins fail."""
    good = oracle.mla_oracle._nearest_even_code

    def bad(a, values):
        a = np.asarray(a, dtype=np.float64)
        if kind == "no_saturation":
            return good(a, values) if np.all(a <= values[-1] * 0.999) else np.full(np.shape(a), len(values))
        hi = np.clip(np.searchsorted(values, a, side="left"), 0, len(values) - 1)
        lo = np.clip(hi - 1, 0, len(values) - 1)
        if kind == "truncate":
            return np.where(values[hi] == a, hi, lo)
        d_lo, d_hi = a - values[lo], values[hi] - a
        return np.where(d_hi <= d_lo, hi, lo)  # ties away from zero

    monkeypatch.setattr(oracle.mla_oracle, "_nearest_even_code", bad)
    failed = 0
    for test in (test_e4m3_quantiser_matches_torch_cast, test_e4m3_quantiser_hand_cases, test_e2m1_quantiser_cases):
        try:
            test()
        except (AssertionError, IndexError):
            failed += 1
    assert failed >= 1


def test_fp8_query_decode_matches_torch():
    """The FP8-query decode (format 3) against torch in float64: the query is cast with
    torch's own float8_e4m3fn (round to nearest even; N(0,1) queries stay far below its
    overflow), the cache codes decoded by torch, then a max-shifted softmax, with the
    causal verify rows of q_len 2."""
    w = gen.make_paged(B=2, H=16, q_len=2, lo=5, hi=90, page_size=32, fmt=gen.FMT_FP8, seed=91, max_blocks=4)
    q, qpe = w.q_f64()
    ro, rl = oracle.paged_decode(q, qpe, w.cache, oracle.FMT_FP8_QFP8, w.kv_scale, w.page_size, w.page_stride,
                                 w.block_tables, w.seq_lens, w.sm_scale)
    f8 = torch.float8_e4m3fn
    for b in range(w.B):
        n = int(w.seq_lens[b])
        pages = [int(w.block_tables[b, i]) for i in range(-(-n // w.page_size))]
        kv = torch.cat([torch.from_numpy(w.cache[p * w.page_stride: p * w.page_stride + w.page_size * 576].copy())
                        .view(f8).to(torch.float64).reshape(w.page_size, 576) for p in pages])[:n] * w.kv_scale
        qt = torch.from_numpy(np.concatenate([q[b], qpe[b]], -1).astype(np.float32)).to(f8).to(torch.float64)
        for i in range(w.q_len):
            vis = n - w.q_len + i + 1
            s = (qt[i] @ kv[:vis].T) * w.sm_scale
            lse = torch.logsumexp(s, -1)
            o = torch.softmax(s, -1) @ kv[:vis, :512]
            assert np.max(np.abs(o.numpy() - ro[b, i])) < 1e-9
            assert np.max(np.abs(lse.numpy() - rl[b, i])) < 1e-9
    # and it is not the bf16-query result
    r1, _ = oracle.paged_decode(q, qpe, w.cache, oracle.FMT_FP8, w.kv_scale, w.page_size, w.page_stride,
                                w.block_tables, w.seq_lens, w.sm_scale)
    assert np.max(np.abs(r1 - ro)) > 1e-4


# ----------------------------------------------------------------------------------
# sliding window and attention sinks (the reading: the window bounds the visible range
# from below; a sink is an extra logit in the denominator with no value)
# ----------------------------------------------------------------------------------

def _ws_workload(fmt=gen.FMT_BF16):
    return gen.make_paged(B=3, H=16, q_len=2, lo=3, hi=150, page_size=32, fmt=fmt, seed=95, max_blocks=5)


def test_window_and_sink_degenerate_cases_equal_plain_attention():
    w = _ws_workload()
    q, qpe = w.q_f64()
    args = (q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables, w.seq_lens, w.sm_scale)
    ro, rl = oracle.paged_decode(*args)
    for window, sinks in ((0, np.full(16, -np.inf)), (int(w.seq_lens.max()) + 5, None)):
        o, l = oracle.paged_decode(*args, window=window, sinks=sinks)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_window_of_one_is_the_query_token():
    # W = 1: query i sees only its own position n - q_len + i: O = that latent row, LSE = its score
    w = _ws_workload()
    q, qpe = w.q_f64()
    o, l = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables,
                               w.seq_lens, w.sm_scale, window=1)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        kv = oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride, w.block_tables[b], n)
        for i in range(w.q_len):
            pos = n - w.q_len + i
            if pos < 0:
                assert np.all(np.isneginf(l[b, i])) and not o[b, i].any()
                continue
            s = w.sm_scale * (q[b, i] @ kv[pos, :512] + qpe[b, i] @ kv[pos, 512:])
            assert np.allclose(o[b, i], kv[pos, :512][None, :], rtol=0, atol=1e-12)
            assert np.allclose(l[b, i], s, rtol=0, atol=1e-12)


def test_sink_closed_form_and_empty_rows():
    # one visible token t and sink sigma: LSE = log(e^s + e^sigma), O = e^(s - LSE) v_t;
    # no visible token: LSE = sigma, O = 0
    qf = np.array([[0.3] * 576])
    kv = np.zeros((3, 576))
    kv[1, :] = 0.01
    s = 0.5 * 0.3 * 0.01 * 576
    o, l = oracle.mla_oracle.attend_window_sink(qf, kv, [1], [2], 0.5, [0.7])
    assert np.isclose(l[0], np.log(np.exp(s) + np.exp(0.7)), rtol=0, atol=1e-14)
    assert np.allclose(o[0], np.exp(s - l[0]) * 0.01, rtol=0, atol=1e-15)
    o, l = oracle.mla_oracle.attend_window_sink(qf, kv, [0], [0], 0.5, [0.7])
    assert l[0] == 0.7 and not o.any()


def test_window_and_sink_match_torch_float64():
    """A banded causal mask and a sink column (zero value) through torch's float64 softmax."""
    w = _ws_workload(gen.FMT_FP8)
    q, qpe = w.q_f64()
    rng = np.random.default_rng(4)
    sinks = rng.standard_normal(16) * 2
    for window in (1, 7, 40):
        ro, rl = oracle.paged_decode(q, qpe, w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                     w.block_tables, w.seq_lens, w.sm_scale, window=window, sinks=sinks)
        for b in range(w.B):
            n = int(w.seq_lens[b])
            kv = torch.from_numpy(oracle.gather_request(w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                                        w.block_tables[b], n))
            qt = torch.from_numpy(np.concatenate([q[b], qpe[b]], -1))  # [q_len, H, 576]
            for i in range(w.q_len):
                pos = n - w.q_len + i
                t = torch.arange(n)
                band = (t <= pos) & (t > pos - window)
                sc = (qt[i] @ kv.T) * w.sm_scale  # [H, n]
                sc = torch.where(band[None, :], sc, torch.tensor(-np.inf, dtype=torch.float64))
                full = torch.cat([sc, torch.from_numpy(sinks)[:, None]], 1)
                lse = torch.logsumexp(full, -1)
                o = torch.softmax(full, -1)[:, :n] @ kv[:, :512]
                assert np.max(np.abs(o.numpy() - ro[b, i])) < 1e-10, (window, b, i)
                assert np.max(np.abs(lse.numpy() - rl[b, i])) < 1e-10, (window, b, i)


@pytest.mark.parametrize("kind", ["window_off_by_one", "sink_in_value", "sink_ignored"])
def test_window_sink_pins_catch_planted_mistakes(kind, monkeypatch):
    """Plant a plausible mistake in a copy of attend_window_sink and check that the torch
    pin or a closed-form pin fails."""
    good = oracle.mla_oracle.attend_window_sink

    def bad(qfull, kv, first, visible, sm_scale, sink):
        first = np.asarray(first)
        sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), (np.asarray(qfull).shape[0],))
        if kind == "window_off_by_one":
            return good(qfull, kv, np.maximum(first - 1, 0), visible, sm_scale, sink)
        if kind == "sink_ignored":
            return good(qfull, kv, first, visible, sm_scale, np.full_like(sink, -np.inf))
        O, lse = good(qfull, kv, first, visible, sm_scale, sink)  # sink_in_value: sink row adds v = 1
        return O + np.where(np.isfinite(sink), np.exp(sink - lse), 0.0)[:, None], lse

    monkeypatch.setattr(oracle.mla_oracle, "attend_window_sink", bad)
    failed = 0
    for test in (test_window_and_sink_match_torch_float64, test_window_of_one_is_the_query_token,
                 test_sink_closed_form_and_empty_rows):
        try:
            test()
        except AssertionError:
            failed += 1
    assert failed >= 1

