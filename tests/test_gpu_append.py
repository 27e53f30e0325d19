"""GPU parity of the cache append (mla_kv_append) against the oracle's kv_append: the
whole page pool must match byte for byte (bit-exact integer and encoding work), on
random rows, on hand-built rows that hit every rounding tie and saturation case, and as
the producer of a cache that the decode then reads."""

import numpy as np
import pytest
import torch

import oracle
import mla_split_kv_02_amd as mla
from workloads import gen
from gpu_util import TOL_LSE, TOL_O_BF16, TOL_O_QUANT, bf16_dev, host, i32_dev, max_err, say, u8_dev

pytestmark = pytest.mark.gpu

FORMATS = [gen.FMT_BF16, gen.FMT_FP8, gen.FMT_NVFP4, oracle.FMT_FP8_QFP8]  # format 3: FP8 pages


def _append_gpu(cache, bits, slots, fmt, kv_scale, page_size, stride):
    c = u8_dev(cache)
    mla.kv_append(bf16_dev(np.ascontiguousarray(bits[:, :512])), bf16_dev(np.ascontiguousarray(bits[:, 512:])),
                  i32_dev(slots), c, fmt, page_size, stride, kv_scale)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def _append_ref(cache, bits, slots, fmt, kv_scale, page_size, stride, num_pages):
    return oracle.kv_append(cache, bits[:, :512], bits[:, 512:], slots, fmt, kv_scale, page_size, stride, num_pages)


def _same_bytes(got, want):
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}"


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("page_size", [32, 64])
def test_append_matches_oracle_bytes(fmt, page_size):
    say(f"append fmt={fmt} page={page_size}")
    rng = np.random.default_rng(70 + 3 * fmt + page_size)
    num_pages = 23
    stride = page_size * oracle.page_row_bytes(fmt) + (48 if page_size == 32 else 0)
    cache = rng.integers(0, 256, num_pages * stride, dtype=np.uint8)
    T = 301
    slots = rng.permutation(num_pages * page_size)[:T].astype(np.int32)
    slots[::37] = -1                       # padding tokens
    slots[5] = num_pages * page_size       # past the pool: skipped
    slots[6] = np.iinfo(np.int32).max
    x = rng.standard_normal((T, oracle.ROW)).astype(np.float32) * 3
    x[7] *= 1000                           # FP8 saturation
    x[8] *= 1e-4                           # subnormal E4M3 codes, zero NVFP4 scales
    bits = gen.to_bf16_bits(x)
    kv_scale = 0.0213
    got = _append_gpu(cache, bits, slots, fmt, kv_scale, page_size, stride)
    _same_bytes(got, _append_ref(cache, bits, slots, fmt, kv_scale, page_size, stride, num_pages))


def test_append_fp8_ties_saturation_and_signed_zero():
    # kv_scale = 1, so x / kv_scale = x: every midpoint between adjacent E4M3 values
    # (exact in bf16), its bf16 neighbours, saturation and signed zeros
    say("append fp8 edge values")
    v = oracle.decode_e4m3fn(np.arange(0x7F))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    mb = gen.to_bf16_bits(mids)
    vals = np.concatenate([mb, mb + 1, mb - 1, mb | 0x8000, (mb + 1) | 0x8000]).astype(np.uint16)
    extra = gen.to_bf16_bits(np.float32([448, 449, 464, 1000, 1e30, -1e30, 0.0, 2 ** -20, -(2 ** -20)]))
    extra = np.concatenate([extra, np.array([0x8000], dtype=np.uint16)])
    vals = np.concatenate([vals, extra])
    T = -(-vals.size // oracle.ROW)
    bits = np.zeros(T * oracle.ROW, dtype=np.uint16)
    bits[:vals.size] = vals
    bits = bits.reshape(T, oracle.ROW)
    page_size, num_pages = 64, 2
    stride = page_size * oracle.ROW
    cache = np.zeros(num_pages * stride, dtype=np.uint8)
    slots = np.arange(T, dtype=np.int32) * 3
    got = _append_gpu(cache, bits, slots, gen.FMT_FP8, 1.0, page_size, stride)
    _same_bytes(got, _append_ref(cache, bits, slots, gen.FMT_FP8, 1.0, page_size, stride, num_pages))


def test_append_nvfp4_ties_and_scales():
    # group layouts with amax = 6 (scale exactly 1, so the codes see the values as they
    # are): every E2M1 midpoint; amax / 6 on an E4M3 midpoint (scale tie); a zero group; a
    # group whose scale rounds to zero; a saturating scale
    say("append nvfp4 edge values")
    g_ties = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -5, 0, -0.0, 0.1, -6, 4, 3]
    g_scale_tie = [6.375, 1, 2, 3, -4, 5, 0.5, 0.25, 1.5, -1.5, 0.75, 6, -6, 0.3, 0.7, 2.2]
    g_zero = [0.0] * 16
    g_tiny = [0.005, -0.003] + [0.001] * 14
    g_huge = [3000, -2999, 1500, 700, 100, 10, 1, 0.1] + [0.0] * 8
    rows = []
    groups = [g_ties, g_scale_tie, g_zero, g_tiny, g_huge]
    for r in range(4):
        row = [groups[(r + k) % len(groups)] for k in range(36)]
        rows.append(np.array(row, dtype=np.float32).reshape(oracle.ROW))
    bits = gen.to_bf16_bits(np.stack(rows))
    bits[:, 11] = 0x8000  # exact negative zero
    page_size, num_pages = 32, 1
    stride = page_size * oracle.page_row_bytes(gen.FMT_NVFP4)
    cache = np.full(num_pages * stride, 0x5A, dtype=np.uint8)
    slots = np.array([0, 31, 5, 17], dtype=np.int32)
    got = _append_gpu(cache, bits, slots, gen.FMT_NVFP4, 1.0, page_size, stride)
    _same_bytes(got, _append_ref(cache, bits, slots, gen.FMT_NVFP4, 1.0, page_size, stride, num_pages))


@pytest.mark.parametrize("fmt", FORMATS)
def test_append_then_decode(fmt):
    # a cache written only by the append kernel, read back by the paged decode
    say(f"append then decode fmt={fmt}")
    rng = np.random.default_rng(80 + fmt)
    page_size, B, H = 64, 3, 16
    seq = np.array([100, 1, 200], dtype=np.int32)
    npg = [-(-int(n) // page_size) for n in seq]
    num_pages = sum(npg) + 2
    perm = rng.permutation(num_pages)
    bt = np.zeros((B, max(npg)), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    stride = page_size * oracle.page_row_bytes(fmt)
    cache = np.zeros(num_pages * stride, dtype=np.uint8)
    x = rng.standard_normal((int(seq.sum()), oracle.ROW)).astype(np.float32)
    bits = gen.to_bf16_bits(x)
    slots = np.concatenate([bt[b, np.arange(n) // page_size] * page_size + np.arange(n) % page_size
                            for b, n in enumerate(seq)]).astype(np.int32)
    fp8 = fmt in (gen.FMT_FP8, oracle.FMT_FP8_QFP8)
    kv_scale = float(np.float32(np.abs(x).max()) / np.float32(448)) if fp8 else 1.0
    c_gpu = _append_gpu(cache, bits, slots, fmt, kv_scale, page_size, stride)
    c_ref = _append_ref(cache, bits, slots, fmt, kv_scale, page_size, stride, num_pages)
    _same_bytes(c_gpu, c_ref)
    q = gen.to_bf16_bits(rng.standard_normal((B, 1, H, 512)).astype(np.float32))
    qpe = gen.to_bf16_bits(rng.standard_normal((B, 1, H, 64)).astype(np.float32))
    o, lse = mla.paged_decode(bf16_dev(q), bf16_dev(qpe), u8_dev(c_gpu), fmt, i32_dev(bt), i32_dev(seq), page_size,
                              stride, kv_scale, gen.SM_SCALE_192)
    torch.cuda.synchronize()
    qf = gen.bf16_bits_to_f32(q).astype(np.float64)
    qpf = gen.bf16_bits_to_f32(qpe).astype(np.float64)
    ro, rl = oracle.paged_decode(qf, qpf, c_ref, fmt, kv_scale, page_size, stride, bt, seq, gen.SM_SCALE_192)
    assert max_err(host(o), ro) <= (TOL_O_BF16 if fmt == gen.FMT_BF16 else TOL_O_QUANT)  # noqa: E501
    assert max_err(host(lse), rl) <= TOL_LSE
