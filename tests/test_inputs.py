"""Seeded generators: determinism, shapes, the QK RMS-norm recipe and the decode lengths."""

import numpy as np
import torch

from causal_sliding_window_amd import inputs


def test_deterministic_and_seed_order():
    a = inputs.training_inputs(1, 16, 2, 8, "f32", seed=5)
    b = inputs.training_inputs(1, 16, 2, 8, "f32", seed=5)
    for n in ("q", "k", "v", "do"):
        assert torch.equal(a[n], b[n])
    c = inputs.training_inputs(1, 16, 2, 8, "f32", seed=4)
    assert torch.equal(c["k"], a["q"])  # seeds s, s+1, s+2, s+3 for q, k, v, dO


def test_qk_norm_unit_rms_and_bf16():
    x = inputs.training_inputs(2, 64, 3, 128, "bf16", seed=0, qk_norm=True)
    for n in ("q", "k"):
        rms = x[n].float().pow(2).mean(-1).sqrt()
        assert torch.allclose(rms, torch.ones_like(rms), atol=1e-2)
        assert x[n].dtype == torch.bfloat16
    assert x["v"].float().std().item() > 0.9


def test_tiny_config_shapes():
    x = inputs.config_inputs("tiny")
    assert x["q"].shape == (1, 128, 2, 64) and x["q"].dtype == torch.float32


def test_decode_lengths_recipe():
    lens = inputs.decode_lengths(32)
    assert lens.dtype == np.int32 and lens.min() >= 512 and lens.max() <= 4096
    assert int(lens.sum()) == 77675 and int(np.minimum(lens, 1024).sum()) == 31834


def test_small_decode_inputs():
    d = inputs.decode_inputs(4, 3, 64, 100, "bf16", seed=7, lengths=[1, 50, 100, 7])
    assert d["k_cache"].shape == (4, 100, 3, 64) and d["seqlens"].dtype == torch.int32
