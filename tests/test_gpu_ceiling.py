"""The measurement kernels behind the benchmark's on-box ceilings compute what they
claim: the stream read touches every byte once (the XOR of its per-thread results is
the XOR of the buffer's 32-bit words), and the MFMA loops finish with finite sums."""

import numpy as np
import pytest
import torch

from mla_split_kv_02_amd import ceiling
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 * 16 + 48, 3), (8 << 20, 64)])
def test_stream_read_touches_every_word(nbytes, blocks):
    say(f"ceiling stream read {nbytes} B, {blocks} blocks")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).to("cuda:0")
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")
    ceiling.stream_read(buf, out, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("kind", [ceiling.MFMA_BF16, ceiling.MFMA_FP8, ceiling.MFMA_F16])
def test_mfma_loop_runs(kind):
    say(f"ceiling mfma kind {kind}")
    out = torch.full((8 * 4,), float("nan"), dtype=torch.float32, device="cuda:0")
    flops = ceiling.mfma(kind, 10, out, 8)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 10 * 4 * (131072 if kind == ceiling.MFMA_FP8 else 32768)
    assert torch.isfinite(out).all()
