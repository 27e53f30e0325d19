"""Seeded synthetic workloads for absorbed-MLA decode (inputs only, no decode math).

Recipe (shared by the oracle and the HIP library; restated in the design notes):
  * numpy ``default_rng(seed)`` (PCG64); all values are float32 draws from N(0, 1).
  * Contiguous workloads draw, in order: Q [B,H,512], QPE [B,H,64], KV [B,S,512],
    KPE [B,S,64]; each is rounded to bf16 (round-to-nearest-even, torch's cast).
  * Paged workloads draw, in order: seq_lens (uniform integers in [lo, hi], both ends
    included), Q [B,q_len,H,512], QPE [B,q_len,H,64], the physical page pool (every
    row of every page, including the unused tail rows of each request's last page),
    then the page permutation.  The pool holds sum_b cdiv(n_b, page) pages; request b
    owns the next cdiv(n_b, page) entries of the permutation, in logical order.  One
    extra "poison" page (NaN codes) sits after the pool and fills every block-table
    entry past a request's last page, so a read past the sequence shows up as NaN
    while staying in bounds.
  * bf16 cache rows are the rounded draws.  FP8 rows use one per-tensor scale
    s = amax / 448 (float32); codes are round-to-nearest-even casts of clamp(x / s,
    +-448) (torch's float8_e4m3fn cast, which does not saturate on its own).  NVFP4
    rows use, per group of 16 consecutive values, the E4M3 scale s_g = RNE(amax_g / 6)
    and E2M1 codes = round-to-nearest-even(x / s_g), saturating at +-6 (all zero when
    s_g = 0); data bytes hold the even value in the low nibble.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE

FMT_BF16 = 0
FMT_FP8 = 1
FMT_NVFP4 = 2
FMT_NAMES = {FMT_BF16: "bf16", FMT_FP8: "fp8_e4m3", FMT_NVFP4: "nvfp4"}

SM_SCALE_192 = 1.0 / math.sqrt(192.0)

# The five workloads, named by what they are.  seed = 1000 + position (1-based).
WORKLOADS = {
    "contig_b1_h16_s256": dict(kind="contig", B=1, H=16, S=256, kv_len_per_split=128, seed=1001),
    "contig_b4_h16_s4096": dict(kind="contig", B=4, H=16, S=4096, seed=1002),
    "contig_b32_h128_s8192": dict(kind="contig", B=32, H=128, S=8192, seed=1003),
    "paged_fp8_b64_h128_s1k_32k": dict(kind="paged", B=64, H=128, q_len=1, lo=1024, hi=32768,
                                       page_size=64, fmt=FMT_FP8, seed=1004),
    "paged_nvfp4_b128_h128_q2_s2k_64k": dict(kind="paged", B=128, H=128, q_len=2, lo=2048,
                                             hi=65536, page_size=64, fmt=FMT_NVFP4, seed=1005),
}


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


# ----------------------------------------------------------------------------------
# Encoders (input preparation only)
# ----------------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN codes (uint8): clamp to +-448, then torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_codes_to_f32(codes: torch.Tensor) -> torch.Tensor:
    return codes.view(torch.float8_e4m3fn).to(torch.float32)


def encode_nvfp4_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rows [R, 576] float32 -> (data [R, 288] uint8, scales [R, 36] uint8)."""
    R = x.shape[0]
    g = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).reshape(R, ROW // 16, 16)
    amax = g.abs().amax(dim=-1)
    s_codes = (amax / 6.0).clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    s_val = _e4m3_codes_to_f32(s_codes)
    safe = torch.where(s_val > 0, s_val, torch.ones_like(s_val))
    v = torch.where((s_val > 0)[..., None], g / safe[..., None], torch.zeros_like(g))
    mag = v.abs()
    # nearest E2M1 magnitude code, ties to the even code (0, .5, 1, 1.5, 2, 3, 4, 6)
    code = ((mag > 0.25).to(torch.uint8) + (mag >= 0.75).to(torch.uint8)
            + (mag > 1.25).to(torch.uint8) + (mag >= 1.75).to(torch.uint8)
            + (mag > 2.5).to(torch.uint8) + (mag >= 3.5).to(torch.uint8)
            + (mag > 5.0).to(torch.uint8))
    code = code | ((v < 0).to(torch.uint8) << 3)
    code = code.reshape(R, ROW)
    data = (code[:, 0::2] | (code[:, 1::2] << 4)).numpy().astype(np.uint8)
    return data, s_codes.numpy().astype(np.uint8)


def row_bytes(fmt: int) -> int:
    return {FMT_BF16: 2 * ROW, FMT_FP8: ROW, FMT_NVFP4: ROW // 2 + ROW // 16}[fmt]


def encode_pages(x: np.ndarray, fmt: int, page_size: int, page_stride: int, kv_scale: float) -> np.ndarray:
    """Rows [npages*page_size, 576] float32 -> page bytes [npages, page_stride] uint8.
    Bytes between the end of a page's content and its stride are filled with 0xFF."""
    npages = x.shape[0] // page_size
    out = np.full((npages, page_stride), 0xFF, dtype=np.uint8)
    if fmt == FMT_BF16:
        b = to_bf16_bits(x).reshape(npages, page_size * ROW).view(np.uint8)
        out[:, :b.shape[1]] = b
    elif fmt == FMT_FP8:
        c = to_e4m3_codes(x / np.float32(kv_scale)).reshape(npages, page_size * ROW)
        out[:, :c.shape[1]] = c
    elif fmt == FMT_NVFP4:
        d, s = encode_nvfp4_rows(x)
        d = d.reshape(npages, page_size * (ROW // 2))
        s = s.reshape(npages, page_size * (ROW // 16))
        out[:, :d.shape[1]] = d
        out[:, d.shape[1]:d.shape[1] + s.shape[1]] = s
    else:
        raise ValueError(fmt)
    return out


def poison_page_bytes(fmt: int, page_size: int, page_stride: int) -> np.ndarray:
    """One page whose every value decodes to NaN (bf16 0x7FC0, E4M3 0x7F, NVFP4 scales
    0x7F)."""
    out = np.full(page_stride, 0xFF, dtype=np.uint8)
    if fmt == FMT_BF16:
        out[:page_size * 2 * ROW] = np.full(page_size * ROW, 0x7FC0, np.uint16).view(np.uint8)
    elif fmt == FMT_FP8:
        out[:page_size * ROW] = 0x7F
    else:
        out[:page_size * ROW // 2] = 0x22
        out[page_size * ROW // 2: page_size * (ROW // 2 + ROW // 16)] = 0x7F
    return out


# ----------------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------------

@dataclass
class ContigInputs:
    B: int
    H: int
    S: int
    q: np.ndarray      # bf16 bits [B,H,512]
    qpe: np.ndarray    # bf16 bits [B,H,64]
    kv: np.ndarray     # bf16 bits [B,S,512]
    kpe: np.ndarray    # bf16 bits [B,S,64]
    sm_scale: float = SM_SCALE_192

    def f64(self):
        """The same bits as float64 values (for the oracle)."""
        return tuple(bf16_bits_to_f32(a).astype(np.float64) for a in (self.q, self.qpe, self.kv, self.kpe))


def make_contig(B: int, H: int, S: int, seed: int, sm_scale: float = SM_SCALE_192,
                zero_q: bool = False) -> ContigInputs:
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, LATENT), dtype=np.float32)
    qpe = rng.standard_normal((B, H, ROPE), dtype=np.float32)
    kv = rng.standard_normal((B, S, LATENT), dtype=np.float32)
    kpe = rng.standard_normal((B, S, ROPE), dtype=np.float32)
    if zero_q:
        q[:] = 0
        qpe[:] = 0
    return ContigInputs(B, H, S, to_bf16_bits(q), to_bf16_bits(qpe), to_bf16_bits(kv),
                        to_bf16_bits(kpe), sm_scale)


@dataclass
class PagedInputs:
    B: int
    H: int
    q_len: int
    fmt: int
    page_size: int
    page_stride: int
    num_pages: int
    q: np.ndarray             # bf16 bits [B,q_len,H,512]
    qpe: np.ndarray           # bf16 bits [B,q_len,H,64]
    cache: np.ndarray         # uint8 [num_pages * page_stride]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray      # int32 [B]
    kv_scale: float = 1.0
    sm_scale: float = SM_SCALE_192
    poison_page: int = -1
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    def q_f64(self):
        return bf16_bits_to_f32(self.q).astype(np.float64), bf16_bits_to_f32(self.qpe).astype(np.float64)

    def kv_bytes(self) -> int:
        """Bytes of cache rows the decode must read: visible tokens x row bytes."""
        return int(np.sum(self.seq_lens.astype(np.int64))) * row_bytes(self.fmt)


def make_paged(B: int, H: int, q_len: int, lo: int, hi: int, page_size: int, fmt: int, seed: int,
               sm_scale: float = SM_SCALE_192, max_blocks: int | None = None,
               seq_lens=None, page_stride: int | None = None, poison_tail: bool = False,
               chunk_pages: int = 2048) -> PagedInputs:
    """Paged workload (see the module recipe).  ``seq_lens`` overrides the draw (the
    generator still draws and discards them, so the stream position is unchanged)."""
    rng = np.random.default_rng(seed)
    drawn = rng.integers(lo, hi, size=B, endpoint=True)
    n = np.asarray(drawn if seq_lens is None else seq_lens, dtype=np.int64)
    q = rng.standard_normal((B, q_len, H, LATENT), dtype=np.float32)
    qpe = rng.standard_normal((B, q_len, H, ROPE), dtype=np.float32)
    npages_b = np.array([cdiv(int(x), page_size) for x in n], dtype=np.int64)
    pool = int(npages_b.sum())
    rb = row_bytes(fmt)
    stride = page_size * rb if page_stride is None else page_stride
    assert stride >= page_size * rb
    num_pages = pool + 1
    cache = np.empty((num_pages, stride), dtype=np.uint8)
    kv_scale = 1.0
    if fmt == FMT_FP8:
        x = rng.standard_normal((pool * page_size, ROW), dtype=np.float32)
        amax = float(np.abs(x).max()) if x.size else 1.0
        kv_scale = float(np.float32(amax) / np.float32(448.0)) if amax > 0 else 1.0
        for p0 in range(0, pool, chunk_pages):
            p1 = min(pool, p0 + chunk_pages)
            cache[p0:p1] = encode_pages(x[p0 * page_size:p1 * page_size], fmt, page_size, stride, kv_scale)
        del x
    else:
        for p0 in range(0, pool, chunk_pages):
            p1 = min(pool, p0 + chunk_pages)
            x = rng.standard_normal(((p1 - p0) * page_size, ROW), dtype=np.float32)
            cache[p0:p1] = encode_pages(x, fmt, page_size, stride, 1.0)
    cache[pool] = poison_page_bytes(fmt, page_size, stride)
    perm = rng.permutation(pool)
    mb = int(npages_b.max()) if max_blocks is None else max_blocks
    mb = max(mb, 1)
    bt = np.full((B, mb), pool, dtype=np.int32)
    off = 0
    for b in range(B):
        k = int(npages_b[b])
        bt[b, :k] = perm[off:off + k]
        off += k
    if poison_tail:
        pz = poison_page_bytes(fmt, page_size, stride)
        for b in range(B):
            r = int(n[b]) % page_size
            if n[b] == 0 or r == 0:
                continue
            page = int(bt[b, int(npages_b[b]) - 1])
            _poison_rows(cache[page], pz, fmt, page_size, r)
    return PagedInputs(B, H, q_len, fmt, page_size, stride, num_pages, to_bf16_bits(q), to_bf16_bits(qpe),
                       cache.reshape(-1), bt, n.astype(np.int32), kv_scale, sm_scale, pool)


def _poison_rows(page: np.ndarray, pz: np.ndarray, fmt: int, page_size: int, first_row: int):
    """Overwrite rows first_row .. page_size-1 of a page with NaN codes."""
    if fmt in (FMT_BF16, FMT_FP8):
        rb = row_bytes(fmt)
        page[first_row * rb: page_size * rb] = pz[first_row * rb: page_size * rb]
    else:
        d = ROW // 2
        page[first_row * d: page_size * d] = pz[first_row * d: page_size * d]
        s0 = page_size * d
        page[s0 + first_row * 36: s0 + page_size * 36] = pz[s0 + first_row * 36: s0 + page_size * 36]


def make_workload(name: str, **overrides):
    """Build one of the named workloads (with optional overrides of its parameters)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    cfg.pop("kv_len_per_split", None)
    if kind == "contig":
        return make_contig(cfg["B"], cfg["H"], cfg["S"], cfg["seed"])
    return make_paged(cfg["B"], cfg["H"], cfg["q_len"], cfg["lo"], cfg["hi"], cfg["page_size"],
                      cfg["fmt"], cfg["seed"], **{k: v for k, v in cfg.items()
                                                   if k not in ("B", "H", "q_len", "lo", "hi", "page_size",
                                                                "fmt", "seed")})
