"""ctypes binding of libmla_ceiling.so (include/mla_ceiling.h): the measurement kernels
behind the benchmark's on-box ceilings.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
CEILING_LIB_PATH = os.path.join(PKG, "libmla_ceiling.so")

MFMA_BF16 = 0
MFMA_FP8 = 1
MFMA_F16 = 2

# every symbol include/mla_ceiling.h declares
EXPORTED_SYMBOLS = ("mla_ceiling_stream_read", "mla_ceiling_mfma", "mla_ceiling_mfma_flops")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(CEILING_LIB_PATH):
        raise ImportError(f"{CEILING_LIB_PATH} is missing: build it with `python -m mla_split_kv_02_amd.build`")
    L = ctypes.CDLL(CEILING_LIB_PATH)
    vp, c_int, c_size = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.mla_ceiling_stream_read.restype = c_int
    L.mla_ceiling_stream_read.argtypes = [vp, c_size, vp, c_int, vp]
    L.mla_ceiling_mfma.restype = c_int
    L.mla_ceiling_mfma.argtypes = [c_int, c_int, vp, c_int, vp]
    L.mla_ceiling_mfma_flops.restype = ctypes.c_double
    L.mla_ceiling_mfma_flops.argtypes = [c_int]
    _lib = L
    return L


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def stream_read(buf: torch.Tensor, out: torch.Tensor, blocks: int) -> None:
    """Enqueue one read of buf (uint8, 16-byte multiple); out: int32 [blocks * 256]."""
    if out.numel() < blocks * 256 or out.dtype != torch.int32:
        raise ValueError("out must be int32 with blocks * 256 elements")
    r = lib().mla_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                      ctypes.c_void_p(out.data_ptr()), int(blocks), _stream(buf.device))
    if r != 0:
        raise RuntimeError(f"mla_ceiling_stream_read failed ({r})")


def mfma(kind: int, iters: int, out: torch.Tensor, blocks: int) -> float:
    """Enqueue one MFMA loop; returns the flops it performs.  out: float32 [blocks * 4]."""
    if out.numel() < blocks * 4 or out.dtype != torch.float32:
        raise ValueError("out must be float32 with blocks * 4 elements")
    r = lib().mla_ceiling_mfma(int(kind), int(iters), ctypes.c_void_p(out.data_ptr()), int(blocks),
                               _stream(out.device))
    if r != 0:
        raise RuntimeError(f"mla_ceiling_mfma failed ({r})")
    return blocks * 4 * iters * 4 * lib().mla_ceiling_mfma_flops(int(kind))
