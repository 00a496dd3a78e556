"""The measurement kernels behind the measured ceilings: the streaming read
touches every word of its buffer once (its partial sums add up to the sum of
the buffer's 32-bit words), and the int8 MFMA loop runs every step (each wave
reports 128 * iters)."""
import sys

import numpy as np
import pytest
import torch

from quantized_moe_expert_router_amd import moeq

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("nbytes,n_blocks", [(16, 1), (4096 + 48, 3), ((64 << 20) + 16 * 77, 1024),
                                             (1 << 26, 65535)])
def test_ceiling_read_sums_every_word(nbytes, n_blocks):
    say("ceiling read", nbytes, n_blocks)
    rng = np.random.default_rng(nbytes + n_blocks)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.uint8).copy()).cuda()
    out = moeq.moeq_ceiling_read(buf, n_blocks)
    torch.cuda.synchronize()
    got = int(out.cpu().numpy().view(np.uint64).sum(dtype=np.uint64))
    want = int(words.astype(np.uint64).sum(dtype=np.uint64))
    assert got == want


@pytest.mark.parametrize("iters,n_blocks", [(1, 1), (37, 5), (1000, 1024)])
def test_ceiling_mfma_runs_every_step(iters, n_blocks):
    say("ceiling mfma", iters, n_blocks)
    out = moeq.moeq_ceiling_mfma_i8(iters, n_blocks, "cuda")
    torch.cuda.synchronize()
    v = out.cpu().numpy().view(np.uint32)
    assert v.shape == (4 * n_blocks,)
    assert np.all(v == np.uint32((128 * iters) % (1 << 32)))
