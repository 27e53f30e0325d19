"""ctypes loader and thin wrappers for libmla_decode.so.

The wrappers check tensor dtypes, shapes, devices and contiguity, allocate outputs with
torch when the caller passes none, and forward raw pointers, sizes and the current HIP
stream to the C ABI.  No arithmetic of the decode happens here.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE_TOO_SMALL = -3
MLA_ERR_HIP = -4
MLA_ERR_SCRATCH_LIMIT = -5
MLA_NOALLOC_SCRATCH_BYTES = 128 << 20

MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
MLA_KV_NVFP4 = 2
MLA_KV_FP8_E4M3_QFP8 = 3  # FP8 pages, query rounded to E4M3, scores on FP8 matrix cores

LATENT, ROPE, ROW = 512, 64, 576

# every symbol include/mla_decode.h declares
EXPORTED_SYMBOLS = (
    "mla_status_string",
    "mla_device_num_cus",
    "mla_plan_contig",
    "mla_plan_paged",
    "mla_paged_workspace_bytes",
    "mla_decode_splitkv",
    "mla_splitkv_combine",
    "mla_paged_decode_partials",
    "mla_paged_combine",
    "mla_paged_decode",
    "mla_paged_decode_ext",
    "mla_paged_decode_noalloc",
    "mla_plan_paged_splits",
    "mla_paged_splits_workspace_bytes",
    "mla_paged_decode_splits",
    "mla_kv_append",
)


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_split_kv_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_float, c_size, c_i64, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64, ctypes.c_void_p
    pint = ctypes.POINTER(c_int)
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [c_int]
    L.mla_device_num_cus.restype = c_int
    L.mla_device_num_cus.argtypes = [c_int, pint]
    L.mla_plan_contig.restype = c_int
    L.mla_plan_contig.argtypes = [c_int, c_int, c_int, pint, pint]
    L.mla_plan_paged.restype = c_int
    L.mla_plan_paged.argtypes = [c_int, c_int, c_int, c_int, pint]
    L.mla_paged_workspace_bytes.restype = c_size
    L.mla_paged_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.mla_decode_splitkv.restype = c_int
    L.mla_decode_splitkv.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_float, c_int, vp, vp, vp]
    L.mla_splitkv_combine.restype = c_int
    L.mla_splitkv_combine.argtypes = [vp, vp, c_int, c_int, vp, vp, vp]
    L.mla_paged_decode_partials.restype = c_int
    L.mla_paged_decode_partials.argtypes = [vp, vp, vp, c_int, c_float, c_int, c_int, c_i64, vp, c_int, vp, c_int,
                                            c_int, c_int, c_float, c_int, vp, c_size, vp]
    L.mla_paged_combine.restype = c_int
    L.mla_paged_combine.argtypes = [vp, c_size, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp, vp]
    L.mla_paged_decode.restype = c_int
    L.mla_paged_decode.argtypes = [vp, vp, vp, c_int, c_float, c_int, c_int, c_i64, vp, c_int, vp, c_int, c_int,
                                   c_int, c_float, c_int, vp, c_size, vp, vp, vp]
    L.mla_paged_decode_ext.restype = c_int
    L.mla_paged_decode_ext.argtypes = [vp, vp, vp, c_int, c_float, c_int, c_int, c_i64, vp, c_int, vp, c_int, c_int,
                                       c_int, c_float, c_int, vp, c_int, vp, c_size, vp, vp, vp]
    L.mla_paged_decode_noalloc.restype = c_int
    L.mla_paged_decode_noalloc.argtypes = [vp, vp, vp, c_int, c_float, c_int, c_int, c_i64, vp, c_int, vp, c_int,
                                           c_int, c_int, c_float, c_int, vp, vp, vp]
    L.mla_plan_paged_splits.restype = c_int
    L.mla_plan_paged_splits.argtypes = [c_int, c_int, c_int, vp, c_int, pint, pint]
    L.mla_paged_splits_workspace_bytes.restype = c_size
    L.mla_paged_splits_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int]
    L.mla_paged_decode_splits.restype = c_int
    L.mla_paged_decode_splits.argtypes = [vp, vp, vp, c_int, c_float, c_int, c_int, c_i64, vp, c_int, vp, c_int,
                                          c_int, c_int, c_float, c_int, c_int, vp, c_size, vp, vp, vp]
    L.mla_kv_append.restype = c_int
    L.mla_kv_append.argtypes = [vp, vp, vp, c_int, vp, c_int, c_float, c_int, c_int, c_i64, vp]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mla_status_string(status).decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MlaError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------------------------
# host-only calls
# ----------------------------------------------------------------------------------

def device_num_cus(device: int = 0) -> int:
    v = ctypes.c_int()
    _check(lib().mla_device_num_cus(device, ctypes.byref(v)), "mla_device_num_cus")
    return v.value


def plan_contig(num_cus: int, B: int, S_kv: int) -> tuple[int, int]:
    L, ns = ctypes.c_int(), ctypes.c_int()
    _check(lib().mla_plan_contig(num_cus, B, S_kv, ctypes.byref(L), ctypes.byref(ns)), "mla_plan_contig")
    return L.value, ns.value


def plan_paged(num_cus: int, B: int, q_len: int, H: int) -> int:
    g = ctypes.c_int()
    _check(lib().mla_plan_paged(num_cus, B, q_len, H, ctypes.byref(g)), "mla_plan_paged")
    return g.value


def paged_workspace_bytes(B: int, q_len: int, H: int, num_splits: int) -> int:
    return int(lib().mla_paged_workspace_bytes(B, q_len, H, num_splits))


def plan_paged_splits(num_cus: int, B: int, q_len: int, seq_lens_host, page_size: int):
    """Fixed-length paged splits from a host copy of seq_lens: (kv_len_per_split, max_splits)."""
    sl = (ctypes.c_int32 * B)(*[int(x) for x in seq_lens_host])
    L, ns = ctypes.c_int(), ctypes.c_int()
    _check(lib().mla_plan_paged_splits(num_cus, B, q_len, ctypes.cast(sl, ctypes.c_void_p), page_size,
                                       ctypes.byref(L), ctypes.byref(ns)), "mla_plan_paged_splits")
    return L.value, ns.value


def paged_splits_workspace_bytes(B: int, q_len: int, H: int, max_splits: int) -> int:
    return int(lib().mla_paged_splits_workspace_bytes(B, q_len, H, max_splits))


# ----------------------------------------------------------------------------------
# device calls
# ----------------------------------------------------------------------------------

def decode_splitkv(q, qpe, kv, kpe, sm_scale=None, kv_len_per_split=None, o_part=None, lse_part=None,
                   num_cus=None):
    """Contiguous split-KV decode (per-split outputs).  q [B,H,512], qpe [B,H,64],
    kv [B,S,512], kpe [B,S,64] bf16.  Returns (o_part [B,H,NS,512] f32,
    lse_part [B,H,NS] f32, kv_len_per_split)."""
    B, H, _ = q.shape
    S = kv.shape[1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, LATENT))
    _need(qpe, "qpe", torch.bfloat16, (B, H, ROPE), dev)
    _need(kv, "kv", torch.bfloat16, (B, S, LATENT), dev)
    _need(kpe, "kpe", torch.bfloat16, (B, S, ROPE), dev)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(LATENT + ROPE)  # TileGym page, mla_decoding_split_kv default
    if kv_len_per_split is None:
        kv_len_per_split, _ = plan_contig(num_cus or device_num_cus(dev.index or 0), B, S)
    ns = -(-S // kv_len_per_split)
    if o_part is None:
        o_part = torch.empty((B, H, ns, LATENT), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((B, H, ns), dtype=torch.float32, device=dev)
    _need(o_part, "o_part", torch.float32, (B, H, ns, LATENT), dev)
    _need(lse_part, "lse_part", torch.float32, (B, H, ns), dev)
    _check(lib().mla_decode_splitkv(_ptr(q), _ptr(qpe), _ptr(kv), _ptr(kpe), B, H, S, float(sm_scale),
                                    int(kv_len_per_split), _ptr(o_part), _ptr(lse_part), _stream(dev)),
           "mla_decode_splitkv")
    return o_part, lse_part, kv_len_per_split


def splitkv_combine(o_part, lse_part, o=None, lse=None, want_lse=True):
    """Split-K LSE reduce.  o_part [..., NS, 512] f32, lse_part [..., NS] f32 ->
    (o [..., 512] bf16, lse [...] f32 or None)."""
    dev = o_part.device
    lead = tuple(o_part.shape[:-2])
    ns = o_part.shape[-2]
    rows = int(math.prod(lead)) if lead else 1
    _need(o_part, "o_part", torch.float32, lead + (ns, LATENT))
    _need(lse_part, "lse_part", torch.float32, lead + (ns,), dev)
    if o is None:
        o = torch.empty(lead + (LATENT,), dtype=torch.bfloat16, device=dev)
    _need(o, "o", torch.bfloat16, lead + (LATENT,), dev)
    if lse is None and want_lse:
        lse = torch.empty(lead, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, lead, dev)
    _check(lib().mla_splitkv_combine(_ptr(o_part), _ptr(lse_part), rows, ns, _ptr(o), _ptr(lse), _stream(dev)),
           "mla_splitkv_combine")
    return o, lse


def paged_workspace(B, q_len, H, num_splits, device):
    """A workspace tensor of the size mla_paged_decode needs (uninitialised)."""
    n = paged_workspace_bytes(B, q_len, H, num_splits)
    if n == 0:
        raise MlaError(MLA_ERR_INVALID_ARG, "mla_paged_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _paged_inputs(q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride, sm_scale):
    """Checks the paged decode's tensors; returns (B, q_len, H, device, page_stride, sm_scale)."""
    B, q_len, H, _ = q.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, q_len, H, LATENT))
    _need(qpe, "qpe", torch.bfloat16, (B, q_len, H, ROPE), dev)
    _need(kv_cache, "kv_cache", torch.uint8, None, dev)
    _need(block_tables, "block_tables", torch.int32, None, dev)
    _need(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    rb = {MLA_KV_BF16: 2 * ROW, MLA_KV_FP8_E4M3: ROW, MLA_KV_NVFP4: ROW // 2 + ROW // 16,
          MLA_KV_FP8_E4M3_QFP8: ROW}.get(fmt)
    if rb is None:
        raise MlaError(MLA_ERR_UNSUPPORTED, "cache format")
    if page_stride is None:
        page_stride = page_size * rb
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(LATENT + ROPE)
    return B, q_len, H, dev, page_stride, sm_scale


def _outputs(o, lse, want_lse, B, q_len, H, dev):
    if o is None:
        o = torch.empty((B, q_len, H, LATENT), dtype=torch.bfloat16, device=dev)
    _need(o, "o", torch.bfloat16, (B, q_len, H, LATENT), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, q_len, H), dev)
    return o, lse


class PagedCall:
    """Checked, marshalled arguments of one paged decode; ``partials()`` and
    ``combine()`` enqueue its two launches, ``run()`` both through mla_paged_decode."""

    def __init__(self, q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride=None, kv_scale=1.0,
                 sm_scale=None, num_splits=None, workspace=None, o=None, lse=None, want_lse=True, num_cus=None,
                 window=0, sinks=None):
        B, q_len, H, dev, page_stride, sm_scale = _paged_inputs(q, qpe, kv_cache, fmt, block_tables, seq_lens,
                                                                 page_size, page_stride, sm_scale)
        if num_splits is None:
            num_splits = plan_paged(num_cus or device_num_cus(dev.index or 0), B, q_len, H)
        if workspace is None:
            workspace = paged_workspace(B, q_len, H, num_splits, dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        o, lse = _outputs(o, lse, want_lse, B, q_len, H, dev)
        self.dev = dev
        self.o, self.lse, self.workspace = o, lse, workspace
        self.num_splits = num_splits
        self.cache_args = (_ptr(q), _ptr(qpe), _ptr(kv_cache), int(fmt), float(kv_scale),
                           int(kv_cache.numel() // page_stride), int(page_size), int(page_stride),
                           _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), B, q_len, H,
                           float(sm_scale), int(num_splits), _ptr(workspace), workspace.numel())
        self.combine_args = (_ptr(workspace), workspace.numel(), _ptr(seq_lens), B, q_len, H, int(num_splits),
                             int(block_tables.shape[1]), int(page_size), _ptr(o), _ptr(lse))
        if sinks is not None:
            _need(sinks, "sinks", torch.float32, (H,), dev)
        self.window, self.sinks = int(window), sinks
        self._keep = (q, qpe, kv_cache, block_tables, seq_lens, sinks)

    def _plain(self):
        return self.window == 0 and self.sinks is None

    def run(self):
        if self._plain():
            _check(lib().mla_paged_decode(*self.cache_args, self.combine_args[-2], self.combine_args[-1],
                                          _stream(self.dev)), "mla_paged_decode")
        else:  # sliding window and / or sinks
            a = self.cache_args
            _check(lib().mla_paged_decode_ext(*a[:15], self.window, _ptr(self.sinks), *a[15:],
                                              self.combine_args[-2], self.combine_args[-1], _stream(self.dev)),
                   "mla_paged_decode_ext")
        return self.o, self.lse

    def partials(self):
        if not self._plain():
            raise ValueError("the separate launches take no window or sinks; use run()")
        _check(lib().mla_paged_decode_partials(*self.cache_args, _stream(self.dev)), "mla_paged_decode_partials")

    def combine(self):
        if not self._plain():
            raise ValueError("the separate launches take no window or sinks; use run()")
        _check(lib().mla_paged_combine(*self.combine_args, _stream(self.dev)), "mla_paged_combine")
        return self.o, self.lse


def paged_decode(q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride=None, kv_scale=1.0,
                 sm_scale=None, num_splits=None, workspace=None, o=None, lse=None, want_lse=True, num_cus=None,
                 window=0, sinks=None):
    """Paged decode.  q [B,q_len,H,512], qpe [B,q_len,H,64] bf16; kv_cache uint8 page pool
    (num_pages * page_stride bytes); block_tables [B,max_blocks] int32; seq_lens [B] int32
    (device).  Returns (o [B,q_len,H,512] bf16, lse [B,q_len,H] f32 or None)."""
    return PagedCall(q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride, kv_scale, sm_scale,
                     num_splits, workspace, o, lse, want_lse, num_cus, window, sinks).run()


def paged_decode_noalloc(q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride=None, kv_scale=1.0,
                         sm_scale=None, num_splits=None, o=None, lse=None, want_lse=True, num_cus=None):
    """paged_decode through mla_paged_decode_noalloc: the workspace is the library's own
    per-GPU scratch array (no workspace tensor).  Outputs are allocated here when not
    given; the C call itself allocates nothing."""
    B, q_len, H, dev, page_stride, sm_scale = _paged_inputs(q, qpe, kv_cache, fmt, block_tables, seq_lens,
                                                             page_size, page_stride, sm_scale)
    if num_splits is None:
        num_splits = plan_paged(num_cus or device_num_cus(dev.index or 0), B, q_len, H)
    o, lse = _outputs(o, lse, want_lse, B, q_len, H, dev)
    _check(lib().mla_paged_decode_noalloc(_ptr(q), _ptr(qpe), _ptr(kv_cache), int(fmt), float(kv_scale),
                                          int(kv_cache.numel() // page_stride), int(page_size), int(page_stride),
                                          _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), B, q_len,
                                          H, float(sm_scale), int(num_splits), _ptr(o), _ptr(lse), _stream(dev)),
           "mla_paged_decode_noalloc")
    return o, lse


def paged_decode_splits(q, qpe, kv_cache, fmt, block_tables, seq_lens, page_size, page_stride=None, kv_scale=1.0,
                        sm_scale=None, kv_len_per_split=None, max_splits=None, seq_lens_host=None, workspace=None,
                        o=None, lse=None, want_lse=True, num_cus=None):
    """Paged decode with fixed-length splits (mla_paged_decode_splits).  Without
    kv_len_per_split / max_splits they come from mla_plan_paged_splits on seq_lens_host
    (a host copy of seq_lens; read from the device here when not given), and max_splits
    is raised to cover max_blocks * page_size.  The workspace holds the partials:
    o_part [B,q_len,H,max_splits,512] f32, then lse_part [B,q_len,H,max_splits] f32 at
    the next 256-byte boundary.  Returns (o, lse, kv_len_per_split, max_splits)."""
    B, q_len, H, dev, page_stride, sm_scale = _paged_inputs(q, qpe, kv_cache, fmt, block_tables, seq_lens,
                                                             page_size, page_stride, sm_scale)
    max_len = int(block_tables.shape[1]) * int(page_size)
    if kv_len_per_split is None:
        if seq_lens_host is None:
            seq_lens_host = seq_lens.cpu().tolist()
        kv_len_per_split, _ = plan_paged_splits(num_cus or device_num_cus(dev.index or 0), B, q_len,
                                                seq_lens_host, page_size)
    if max_splits is None:
        max_splits = -(-max_len // kv_len_per_split)
    if workspace is None:
        n = paged_splits_workspace_bytes(B, q_len, H, max_splits)
        if n == 0:
            raise MlaError(MLA_ERR_INVALID_ARG, "mla_paged_splits_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    o, lse = _outputs(o, lse, want_lse, B, q_len, H, dev)
    _check(lib().mla_paged_decode_splits(_ptr(q), _ptr(qpe), _ptr(kv_cache), int(fmt), float(kv_scale),
                                         int(kv_cache.numel() // page_stride), int(page_size), int(page_stride),
                                         _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens), B, q_len, H,
                                         float(sm_scale), int(kv_len_per_split), int(max_splits), _ptr(workspace),
                                         workspace.numel(), _ptr(o), _ptr(lse), _stream(dev)),
           "mla_paged_decode_splits")
    return o, lse, kv_len_per_split, max_splits


def kv_append(latent, rope, slots, kv_cache, fmt, page_size, page_stride=None, kv_scale=1.0):
    """Store T new tokens into the page pool in place.  latent [T,512], rope [T,64] bf16;
    slots [T] int32 (page * page_size + row; slots outside the pool are skipped);
    kv_cache uint8 page pool of num_pages * page_stride bytes.  Returns kv_cache."""
    T = latent.shape[0] if latent.dim() == 2 else -1
    dev = kv_cache.device
    _need(latent, "latent", torch.bfloat16, (T, LATENT), dev)
    _need(rope, "rope", torch.bfloat16, (T, ROPE), dev)
    _need(slots, "slots", torch.int32, (T,), dev)
    _need(kv_cache, "kv_cache", torch.uint8, None, dev)
    rb = {MLA_KV_BF16: 2 * ROW, MLA_KV_FP8_E4M3: ROW, MLA_KV_NVFP4: ROW // 2 + ROW // 16,
              MLA_KV_FP8_E4M3_QFP8: ROW}.get(fmt)
    if rb is None:
        raise MlaError(MLA_ERR_UNSUPPORTED, "cache format")
    if page_stride is None:
        page_stride = page_size * rb
    _check(lib().mla_kv_append(_ptr(latent), _ptr(rope), _ptr(slots), T, _ptr(kv_cache), int(fmt), float(kv_scale),
                               int(kv_cache.numel() // page_stride), int(page_size), int(page_stride),
                               _stream(dev)), "mla_kv_append")
    return kv_cache
