"""Plain float64 CPU oracle for absorbed Multi-head Latent Attention (MLA) decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code with
the HIP library and never imports it.  Every function is the textbook definition of
what the decode path computes, written for a reader to check by eye: no blocking,
no online softmax, no fusion.  numpy ``@`` is the only library primitive used.

Sources (three web pages; cited by page and section):
  * TileGym page ``mla_decoding_split_kv.py`` ("CUDA Tile C++ MLA Decoding with
    Split-KV"): the contiguous split-KV op, its planner helpers ``next_power_of_2`` and
    ``cdiv``, the shapes in ``_mla_decoding_split_kv.forward`` (Q [B,H,512], QPE
    [B,H,64], KV [B,S,512], KPE [B,S,64], K = V = KV), the per-split outputs
    ``Att_Out``/``LSE_Out`` and the split-K reduce that merges them.
  * TokenSpeed page ``tokenspeed_mla.py`` ("CuteDSL MLA attention backend"):
    ``forward_decode`` (paged cache viewed as [pages, page_size, 576], query viewed as
    [bs, q_len, H, head_dim], cache row split at ``kv_lora_rank`` into latent and rope,
    FP8 E4M3 cache with its scale folded into the softmax scale) and the module note on
    the decode workspace (D + 1 fp32 values per split).
  * metrale page ``kv_cache_mla.rs``: ``mla_paged_decode_nvfp4`` (a token is 512 + 64 =
    576 values; a page holds packed E2M1 data followed by one E4M3 scale per 16 values)
    and ``mla_paged_decode_fp8`` (scalar dequant scale, byte strides).

Readings where the pages are silent are listed in the repository's design notes; the
ones this module depends on are restated at each function.

Parity status: every public function here is pinned by tests under ``tests/``
(brute force, torch's float64 SDPA, closed forms, invariances, torch's float8 decode
and cast, the OCP MX E2M1 value table, the input recipe's separate encoders, and planted
mistakes that the pins must catch).  That covers the cache append (``quantize_e4m3``,
``quantize_e2m1``, ``encode_row``, ``kv_append``), the FP8-query format and the sliding
window with sinks (``attend_window_sink``).  None is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Cache-row geometry: metrale page, ``mla_paged_decode_nvfp4`` doc comment (512 + 64 =
# 576 values per token); TileGym page, ``forward`` (HEAD_DIM = 512, KPE_DIM = 64).
LATENT = 512
ROPE = 64
ROW = LATENT + ROPE

# Cache formats (the integer codes are this library's, see include/mla_decode.h).
FMT_BF16 = 0
FMT_FP8 = 1
FMT_NVFP4 = 2
FMT_FP8_QFP8 = 3  # FP8 pages; the query is rounded to E4M3 before the scores (see paged_decode_request)

NVFP4_GROUP = 16  # metrale page, ``mla_paged_decode_nvfp4``: one E4M3 scale per 16 values


# ----------------------------------------------------------------------------------
# Planner (integer): TileGym page, helpers and ``forward``
# ----------------------------------------------------------------------------------

def cdiv(a: int, b: int) -> int:
    """Ceiling division (TileGym page, helper ``cdiv``)."""
    return -(-a // b)


def next_power_of_2(n: int) -> int:
    """Smallest power of two that is >= n, and 1 for n <= 0 (TileGym page, helper
    ``next_power_of_2``)."""
    if n <= 0:
        return 1
    p = 1
    while p < n:
        p *= 2
    return p


def plan_contig(num_cus: int, B: int, S_kv: int, tile_n: int = 128) -> tuple[int, int]:
    """Split planner of the TileGym page, ``_mla_decoding_split_kv.forward``.

    estimated splits = max(1, compute units // B); kv_len_per_split =
    max(next_power_of_2(S_kv // estimate), TILE_N) with TILE_N = 128; number of splits =
    cdiv(S_kv, kv_len_per_split).  Returns (kv_len_per_split, num_splits).
    """
    est = max(1, num_cus // B)
    L = max(next_power_of_2(S_kv // est), tile_n)
    return L, cdiv(S_kv, L)


def workspace_floats_per_split(q_len: int, H: int) -> int:
    """Float32 values one split of one request occupies in the decode workspace: the
    normalised partial output (D = 512) plus its log-sum-exp, for every (query, head)
    row (TokenSpeed page, module note on the decode workspace: D + 1 values per split,
    fp32 accumulator)."""
    return q_len * H * (LATENT + 1)


# ----------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------

def decode_e4m3fn(codes) -> np.ndarray:
    """Decode FP8 E4M3 codes to float64 (OCP 8-bit floating point, E4M3 "FN" variant).

    The TokenSpeed page casts with torch's ``float8_e4m3fn``; the metrale page names
    "FP8 E4M3".  Bit layout s.eeee.mmm, exponent bias 7; exponent 0 is subnormal
    (m/8 * 2**-6); s.1111.111 is NaN; there are no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def decode_e2m1(codes) -> np.ndarray:
    """Decode FP4 E2M1 codes (low 4 bits) to float64 (OCP MX E2M1, named by the metrale
    page for the NVFP4 cache).  Bit layout s.ee.m, exponent bias 1; exponent 0 is
    subnormal (m/2); no infinities or NaN.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    subnormal = m / 2.0
    return sign * np.where(e == 0, subnormal, normal)


def decode_bf16_bits(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: the 16 bits are the top half of an
    IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# Paged cache rows
# ----------------------------------------------------------------------------------

def page_row_bytes(fmt: int) -> int:
    """Bytes of one token row inside a page: 576 bf16 values, 576 FP8 codes, or 288
    packed E2M1 bytes plus 36 E4M3 scales (NVFP4)."""
    return {FMT_BF16: 2 * ROW, FMT_FP8: ROW, FMT_NVFP4: ROW // 2 + ROW // NVFP4_GROUP, FMT_FP8_QFP8: ROW}[fmt]


def decode_page(page: np.ndarray, fmt: int, page_size: int, kv_scale: float = 1.0) -> np.ndarray:
    """Decode one page (its bytes, uint8) into float64 rows [page_size, 576].

    * bf16: row-major [page_size][576] bf16 (TokenSpeed page, ``forward_decode``: cache
      viewed as [num_pages, page_size, kv_cache_dim]).
    * FP8: row-major [page_size][576] E4M3 codes; value = kv_scale * e4m3(code)
      (metrale page, ``mla_paged_decode_fp8``: scalar dequant scale; K and V alias one
      cache, so one scale serves both).
    * NVFP4: data section [page_size][288] bytes, two E2M1 codes per byte with the even
      value in the low nibble, then [page_size][36] E4M3 scales, scale g covering values
      16g .. 16g+15 of the row; value = e2m1(code) * e4m3(scale) (metrale page,
      ``mla_paged_decode_nvfp4``: packed E2M1 data followed by one E4M3 scale per 16
      values).
    """
    page = np.asarray(page, dtype=np.uint8)
    if fmt == FMT_BF16:
        bits = page[: page_size * 2 * ROW].view(np.uint16).reshape(page_size, ROW)
        return decode_bf16_bits(bits)
    if fmt in (FMT_FP8, FMT_FP8_QFP8):
        codes = page[: page_size * ROW].reshape(page_size, ROW)
        return kv_scale * decode_e4m3fn(codes)
    if fmt == FMT_NVFP4:
        data_bytes = ROW // 2
        data = page[: page_size * data_bytes].reshape(page_size, data_bytes).astype(np.int64)
        codes = np.empty((page_size, ROW), dtype=np.int64)
        codes[:, 0::2] = data & 0xF
        codes[:, 1::2] = data >> 4
        sc_off = page_size * data_bytes
        ngroups = ROW // NVFP4_GROUP
        scales = decode_e4m3fn(page[sc_off: sc_off + page_size * ngroups].reshape(page_size, ngroups))
        return decode_e2m1(codes) * np.repeat(scales, NVFP4_GROUP, axis=1)
    raise ValueError(f"unknown cache format {fmt}")


def gather_request(cache: np.ndarray, fmt: int, kv_scale: float, page_size: int, page_stride: int,
                   block_row: np.ndarray, n: int) -> np.ndarray:
    """Logical cache rows [n, 576] of one request: token t lives in row t % page_size of
    page block_row[t // page_size] (TokenSpeed page, ``forward_decode`` and the
    block-table metadata; metrale page, ``block_tables``/``seq_lens``/``block_size``).
    Table entries past cdiv(n, page_size) are never read."""
    if n == 0:
        return np.zeros((0, ROW))
    rows = []
    for i in range(cdiv(n, page_size)):
        p = int(block_row[i])
        rows.append(decode_page(cache[p * page_stride:(p + 1) * page_stride], fmt, page_size, kv_scale))
    return np.concatenate(rows, axis=0)[:n]


# ----------------------------------------------------------------------------------
# Attention: the plain definition
# ----------------------------------------------------------------------------------

def attend(qfull: np.ndarray, kv: np.ndarray, visible, sm_scale: float):
    """Absorbed-MLA attention of R query rows over n cache rows, in float64.

    qfull: [R, 576] = [Q | QPE];  kv: [n, 576] = [latent | rope];  visible: [R] ints,
    row r attends tokens 0 .. visible[r]-1.

    score s[r, t] = sm_scale * (Q[r] . latent[t] + QPE[r] . rope[t]);
    lse[r] = log sum_t exp(s[r, t]);  O[r] = sum_t exp(s[r, t] - lse[r]) * latent[t].
    K and V alias one latent (TileGym page, ``forward``: "K=V=KV"), so V is the 512-wide
    latent.  A row with no visible token gets lse = -inf and O = 0.
    """
    qfull = np.asarray(qfull, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    R, n = qfull.shape[0], kv.shape[0]
    visible = np.broadcast_to(np.asarray(visible, dtype=np.int64), (R,))
    O = np.zeros((R, LATENT))
    lse = np.full(R, -np.inf)
    if n == 0:
        return O, lse
    s = sm_scale * (qfull[:, :LATENT] @ kv[:, :LATENT].T + qfull[:, LATENT:] @ kv[:, LATENT:].T)
    for r in range(R):
        v = int(min(max(visible[r], 0), n))
        if v == 0:
            continue
        sr = s[r, :v]
        m = sr.max()
        lse[r] = m + math.log(np.exp(sr - m).sum())
        O[r] = np.exp(sr - lse[r]) @ kv[:v, :LATENT]
    return O, lse


def attend_window_sink(qfull: np.ndarray, kv: np.ndarray, first, visible, sm_scale: float, sink):
    """``attend`` with a lower bound and a sink: row r attends tokens first[r] ..
    visible[r]-1, and sink[r] (a logit in the units of the scaled scores, -inf for none)
    joins the softmax denominator only:
        lse[r] = log(exp(sink[r]) + sum_t exp(s[r, t]));  O[r] = sum_t exp(s[r, t] - lse[r]) * latent[t].
    metrale page, ``mla_paged_decode_fp8``: a ``sliding_window`` argument and per-head fp32
    ``sinks`` (may be null).  The page does not define them; this is the reading that the
    window bounds the visible range from below and a sink is an extra logit with no value.
    """
    qfull = np.asarray(qfull, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    R, n = qfull.shape[0], kv.shape[0]
    first = np.broadcast_to(np.asarray(first, dtype=np.int64), (R,))
    visible = np.broadcast_to(np.asarray(visible, dtype=np.int64), (R,))
    sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), (R,))
    O = np.zeros((R, LATENT))
    lse = np.full(R, -np.inf)
    s = sm_scale * (qfull[:, :LATENT] @ kv[:, :LATENT].T + qfull[:, LATENT:] @ kv[:, LATENT:].T) if n else None
    for r in range(R):
        hi = int(min(max(visible[r], 0), n))
        lo = int(min(max(first[r], 0), hi))
        terms = [] if hi == lo else list(s[r, lo:hi])
        if sink[r] != -np.inf:
            terms.append(sink[r])
        if not terms:
            continue
        t = np.array(terms)
        m = t.max()
        lse[r] = m + math.log(np.exp(t - m).sum())
        if hi > lo:
            O[r] = np.exp(s[r, lo:hi] - lse[r]) @ kv[lo:hi, :LATENT]
    return O, lse


def attend_range(qfull, kv, visible, sm_scale, start: int, stop: int):
    """Split partial: ``attend`` restricted to tokens [start, stop).  Returns the
    normalised partial output O_j and its lse_j; an empty range (or one this row cannot
    see) gives lse_j = -inf and O_j = 0 (TileGym page, ``forward``: each split writes a
    partial output and an fp32 LSE)."""
    visible = np.asarray(visible, dtype=np.int64)
    vis_local = np.clip(visible - start, 0, max(stop - start, 0))
    return attend(qfull, kv[start:stop], vis_local, sm_scale)


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Split-K log-sum-exp reduce (TileGym page, ``forward``: ``splitk_reduce`` merges
    ``Att_Out``/``LSE_Out`` into O).

    o_parts [R, NS, 512] normalised partials, lse_parts [R, NS].
    M = max_j lse_j; LSE = M + log sum_j exp(lse_j - M); O = sum_j exp(lse_j - LSE) O_j.
    Splits with lse_j = -inf contribute nothing; if all are -inf, O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    R = lse_parts.shape[0]
    O = np.zeros((R, o_parts.shape[-1]))
    LSE = np.full(R, -np.inf)
    for r in range(R):
        live = np.isfinite(lse_parts[r])
        if not live.any():
            continue
        lj = lse_parts[r, live]
        M = lj.max()
        LSE[r] = M + math.log(np.exp(lj - M).sum())
        O[r] = np.exp(lj - LSE[r]) @ o_parts[r, live]
    return O, LSE


# ----------------------------------------------------------------------------------
# Contiguous split-KV decode (TileGym page)
# ----------------------------------------------------------------------------------

def _qfull(q, qpe):
    return np.concatenate([np.asarray(q, np.float64), np.asarray(qpe, np.float64)], axis=-1)


def contig_decode_splitkv(q, qpe, kv, kpe, sm_scale: float, kv_len_per_split: int):
    """Per-split outputs of the contiguous op (TileGym page, ``forward``).

    q [B,H,512], qpe [B,H,64], kv [B,S,512], kpe [B,S,64] (float64 values).
    Split j covers tokens [j*L, min((j+1)*L, S)) with L = kv_len_per_split and
    NS = cdiv(S, L).  Returns Att_Out [B,H,NS,512] (normalised partials, float64) and
    LSE_Out [B,H,NS].
    """
    q = np.asarray(q, np.float64)
    B, H, _ = q.shape
    S = np.asarray(kv).shape[1]
    L = kv_len_per_split
    NS = cdiv(S, L)
    o_part = np.zeros((B, H, NS, LATENT))
    lse_part = np.full((B, H, NS), -np.inf)
    qf = _qfull(q, qpe)
    for b in range(B):
        rows = np.concatenate([np.asarray(kv[b], np.float64), np.asarray(kpe[b], np.float64)], axis=-1)
        for j in range(NS):
            o, l = attend_range(qf[b], rows, np.full(H, S), sm_scale, j * L, min((j + 1) * L, S))
            o_part[b, :, j] = o
            lse_part[b, :, j] = l
    return o_part, lse_part


def contig_decode(q, qpe, kv, kpe, sm_scale: float):
    """Final output of the contiguous op: O [B,H,512] and LSE [B,H] over all S tokens."""
    q = np.asarray(q, np.float64)
    B, H, _ = q.shape
    S = np.asarray(kv).shape[1]
    qf = _qfull(q, qpe)
    O = np.zeros((B, H, LATENT))
    LSE = np.zeros((B, H))
    for b in range(B):
        rows = np.concatenate([np.asarray(kv[b], np.float64), np.asarray(kpe[b], np.float64)], axis=-1)
        O[b], LSE[b] = attend(qf[b], rows, np.full(H, S), sm_scale)
    return O, LSE


# ----------------------------------------------------------------------------------
# Paged decode (TokenSpeed page ``forward_decode``; metrale page paged launchers)
# ----------------------------------------------------------------------------------

def visible_counts(n: int, q_len: int) -> np.ndarray:
    """Tokens query i of a request sees: the cache already holds the q_len new tokens
    (TokenSpeed page, ``forward_decode`` writes the cache before attention), query i sits
    at position n - q_len + i and sees tokens 0 .. n - q_len + i (causal across the
    draft tokens).  For q_len = 1 this is all n tokens."""
    return np.array([max(n - q_len + i + 1, 0) for i in range(q_len)], dtype=np.int64)


def paged_decode_request(q_b, qpe_b, cache, fmt: int, kv_scale: float, page_size: int,
                         page_stride: int, block_row, n: int, sm_scale: float, heads=None,
                         window: int = 0, sinks=None):
    """One request of the paged op.  q_b [q_len,H,512], qpe_b [q_len,H,64] (float64
    values).  Returns O [q_len,H',512] and LSE [q_len,H'] for the chosen heads (all by
    default).

    FMT_FP8_QFP8: TokenSpeed page, ``forward_decode``: with an FP8 cache the query is
    cast to the cache's FP8 type before the kernel (and k_scale goes into the softmax
    scale, which is what scoring against kv_scale * e4m3(code) computes).  The query and
    its rope part are rounded to E4M3 here (quantize_e4m3: nearest, ties to even,
    saturating at 448); everything after is the same definition."""
    q_b = np.asarray(q_b, np.float64)
    qpe_b = np.asarray(qpe_b, np.float64)
    if fmt == FMT_FP8_QFP8:
        q_b = decode_e4m3fn(quantize_e4m3(q_b.astype(np.float32)))
        qpe_b = decode_e4m3fn(quantize_e4m3(qpe_b.astype(np.float32)))
    q_len, H, _ = q_b.shape
    hs = np.arange(H) if heads is None else np.asarray(heads)
    kv = gather_request(cache, fmt, kv_scale, page_size, page_stride, block_row, n)
    vis = visible_counts(n, q_len)
    qf = _qfull(q_b[:, hs], qpe_b[:, hs]).reshape(q_len * len(hs), ROW)
    if window == 0 and sinks is None:
        O, LSE = attend(qf, kv, np.repeat(vis, len(hs)), sm_scale)
    else:
        # window W > 0: query i (position n - q_len + i) sees its last W tokens
        first = np.maximum(vis - window, 0) if window > 0 else np.zeros_like(vis)
        sk = np.full(len(hs), -np.inf) if sinks is None else np.asarray(sinks, np.float64)[hs]
        O, LSE = attend_window_sink(qf, kv, np.repeat(first, len(hs)), np.repeat(vis, len(hs)), sm_scale,
                                    np.tile(sk, q_len))
    return O.reshape(q_len, len(hs), LATENT), LSE.reshape(q_len, len(hs))


def paged_decode(q, qpe, cache, fmt: int, kv_scale: float, page_size: int, page_stride: int,
                 block_tables, seq_lens, sm_scale: float, requests=None, heads=None, window: int = 0,
                 sinks=None):
    """Paged absorbed-MLA decode.  q [B,q_len,H,512], qpe [B,q_len,H,64]; cache is the
    raw page pool (uint8, num_pages * page_stride bytes); block_tables [B, max_blocks]
    int; seq_lens [B] int.  Returns O [B',q_len,H',512] and LSE [B',q_len,H'] for the
    chosen requests and heads (all by default)."""
    bs = range(len(seq_lens)) if requests is None else requests
    outs, lses = [], []
    for b in bs:
        o, l = paged_decode_request(q[b], qpe[b], cache, fmt, kv_scale, page_size, page_stride,
                                    block_tables[b], int(seq_lens[b]), sm_scale, heads, window, sinks)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def paged_decode_split_partials(q, qpe, cache, fmt: int, kv_scale: float, page_size: int, page_stride: int,
                                block_tables, seq_lens, sm_scale: float, kv_len_per_split: int, num_splits: int):
    """Per-split partials of the paged op with fixed-length splits (TileGym page,
    ``forward``: split j of a sequence covers tokens [j*L, (j+1)*L) with L =
    kv_len_per_split, each writing a normalised partial and its LSE; TokenSpeed page,
    ``forward_decode``: the query rows and the paged cache).  A request of n tokens
    clips split j to [j*L, min((j+1)*L, n)); splits past n, and rows that see no token
    of a split (q_len > 1), are empty: O_j = 0, lse_j = -inf.  Returns o_part
    [B,q_len,H,NS,512] and lse_part [B,q_len,H,NS] (float64)."""
    q = np.asarray(q, np.float64)
    qpe = np.asarray(qpe, np.float64)
    if fmt == FMT_FP8_QFP8:
        q = decode_e4m3fn(quantize_e4m3(q.astype(np.float32)))
        qpe = decode_e4m3fn(quantize_e4m3(qpe.astype(np.float32)))
    B, q_len, H, _ = q.shape
    L, NS = kv_len_per_split, num_splits
    o_part = np.zeros((B, q_len, H, NS, LATENT))
    lse_part = np.full((B, q_len, H, NS), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        kv = gather_request(cache, fmt, kv_scale, page_size, page_stride, block_tables[b], n)
        vis = np.repeat(visible_counts(n, q_len), H)
        qf = _qfull(q[b], qpe[b]).reshape(q_len * H, ROW)
        for j in range(NS):
            lo, hi = min(j * L, n), min((j + 1) * L, n)
            o, l = attend_range(qf, kv, vis, sm_scale, lo, hi)
            o_part[b, :, :, j] = o.reshape(q_len, H, LATENT)
            lse_part[b, :, :, j] = l.reshape(q_len, H)
    return o_part, lse_part


# ----------------------------------------------------------------------------------
# KV-cache append: the write that precedes the decode
# ----------------------------------------------------------------------------------
#
# TokenSpeed page, ``forward_decode``: before attending, the new tokens' latent
# (k[..., :kv_lora_rank]) and rope key (k[..., kv_lora_rank:]) are stored into the
# paged pool at their cache locations (``set_mla_kv_buffer`` with ``out_cache_loc``);
# the pool holds the cache dtype (FP8 E4M3 for that backend).  metrale page,
# ``mla_cache_assemble``: one token's cache row is [kv_latent | k_rope].  The pages do
# not spell out the quantisation; the readings used here are the same as the input
# recipe's: FP8 code = nearest E4M3 value of x / kv_scale after saturation at +-448,
# ties to the even code; NVFP4 scale = nearest E4M3 value of amax/6 (saturated at 448),
# data = nearest E2M1 value of x / scale (saturated at +-6), ties to the even code, all
# zeros when the scale is zero.  The sign of the scaled value is kept (so a negative
# value that rounds to zero gives the negative-zero code).  Divisions are binary32.

def _e4m3_positive_values() -> np.ndarray:
    """Values of the non-negative finite E4M3 codes 0x00 .. 0x7E, in code order (which
    is increasing value order)."""
    return decode_e4m3fn(np.arange(0x7F))


def _e2m1_positive_values() -> np.ndarray:
    """Values of the non-negative E2M1 codes 0 .. 7, in code order."""
    return decode_e2m1(np.arange(8))


def _nearest_even_code(a: np.ndarray, values: np.ndarray) -> np.ndarray:
    """For magnitudes a (float64, 0 <= a <= values[-1]), the index of the nearest entry
    of the increasing table `values`; on a tie the even index (even mantissa) wins."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(values, a, side="left"), 0, len(values) - 1)
    lo = np.clip(hi - 1, 0, len(values) - 1)
    d_lo = a - values[lo]
    d_hi = values[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def quantize_e4m3(y) -> np.ndarray:
    """binary32 values -> E4M3 codes (uint8): saturate at +-448, nearest value, ties to
    the even code, sign of y kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    mag = _nearest_even_code(a, _e4m3_positive_values()).astype(np.uint8)
    return np.where(np.signbit(y), mag | 0x80, mag).astype(np.uint8)


def quantize_e2m1(y) -> np.ndarray:
    """binary32 values -> E2M1 codes (low 4 bits of uint8): saturate at +-6, nearest
    value, ties to the even code, sign of y kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 6.0)
    mag = _nearest_even_code(a, _e2m1_positive_values()).astype(np.uint8)
    return np.where(np.signbit(y), mag | 0x8, mag).astype(np.uint8)


def encode_row(row_bits: np.ndarray, fmt: int, kv_scale: float = 1.0) -> np.ndarray:
    """One cache row (576 bf16 bit patterns: latent then rope) -> its bytes in the page
    format.  bf16: the bit patterns themselves.  FP8: 576 codes of x / kv_scale.
    NVFP4: (288 data bytes, 36 scale codes) returned concatenated."""
    row_bits = np.asarray(row_bits, dtype=np.uint16).reshape(ROW)
    if fmt == FMT_BF16:
        return row_bits.view(np.uint8).copy()
    x = decode_bf16_bits(row_bits).astype(np.float32)  # exact
    if fmt in (FMT_FP8, FMT_FP8_QFP8):  # the same page bytes
        y = x / np.float32(kv_scale)
        return quantize_e4m3(y)
    if fmt == FMT_NVFP4:
        g = x.reshape(ROW // NVFP4_GROUP, NVFP4_GROUP)
        amax = np.abs(g).max(axis=1)
        s_code = quantize_e4m3(amax / np.float32(6.0))
        s_val = decode_e4m3fn(s_code).astype(np.float32)
        codes = np.zeros_like(g, dtype=np.uint8)
        for i in range(g.shape[0]):
            if s_val[i] > 0:
                codes[i] = quantize_e2m1(g[i] / s_val[i])
        codes = codes.reshape(ROW)
        data = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
        return np.concatenate([data, s_code])
    raise ValueError(f"unknown cache format {fmt}")


def kv_append(cache: np.ndarray, latent_bits, rope_bits, slots, fmt: int, kv_scale: float,
              page_size: int, page_stride: int, num_pages: int) -> np.ndarray:
    """Returns a copy of the page pool (uint8 bytes) with token j's row [latent_j |
    rope_j] stored at flat slot slots[j] = page * page_size + row.  Slots outside
    [0, num_pages * page_size) are skipped.  NVFP4: the 288 data bytes go to the page's
    data section at row * 288, the 36 scales to its scale section (after page_size *
    288 data bytes) at row * 36, as decode_page reads them."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    latent_bits = np.asarray(latent_bits, dtype=np.uint16).reshape(-1, LATENT)
    rope_bits = np.asarray(rope_bits, dtype=np.uint16).reshape(-1, ROPE)
    for j, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0 or slot >= num_pages * page_size:
            continue
        page, r = divmod(int(slot), page_size)
        base = page * page_stride
        enc = encode_row(np.concatenate([latent_bits[j], rope_bits[j]]), fmt, kv_scale)
        if fmt == FMT_NVFP4:
            d, s = enc[: ROW // 2], enc[ROW // 2:]
            out[base + r * (ROW // 2): base + (r + 1) * (ROW // 2)] = d
            sc = base + page_size * (ROW // 2) + r * (ROW // NVFP4_GROUP)
            out[sc: sc + ROW // NVFP4_GROUP] = s
        else:
            nb = page_row_bytes(fmt)
            out[base + r * nb: base + (r + 1) * nb] = enc
    return out
