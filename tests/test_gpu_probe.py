"""GPU checks of the measurement probes (swattn_probe_mfma, swattn_probe_read): the
values they compute are exact, so the timed work is the work described."""

import numpy as np
import pytest
import torch

from causal_sliding_window_amd import swattn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (64, 1000), (512, 4096)])
def test_probe_mfma_products_are_exact(workgroups, iters):
    """All operands are 1/256, so every output element is iters / 64 exactly."""
    out = torch.full((workgroups * 256,), -1.0, dtype=torch.float32, device=DEV)
    swattn.swattn_probe_mfma(out, workgroups, iters)
    torch.cuda.synchronize()
    assert torch.all(out == iters / 64)


@pytest.mark.parametrize("words,workgroups", [(4, 1), ((1 << 20) + 4, 7), ((1 << 22) + 36, 1024)])
def test_probe_read_xor_covers_every_word(words, workgroups):
    """The XOR of the per-thread words equals the XOR of the buffer: every 16-byte piece
    is read exactly once, also in the ragged tail of the grid stride."""
    g = torch.Generator().manual_seed(words)
    src = torch.randint(-(2 ** 31), 2 ** 31 - 1, (words,), dtype=torch.int32, generator=g)
    out = torch.zeros(workgroups * 256, dtype=torch.int32, device=DEV)
    swattn.swattn_probe_read(src.to(DEV), out, workgroups)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(out.cpu().numpy()) == np.bitwise_xor.reduce(src.numpy())
