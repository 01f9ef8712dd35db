"""The allocation-free decode entry point (swattn_decode_noalloc) through the C ABI,
against swattn_decode on the same inputs: the same kernels, so the outputs must be
bitwise equal.  Two calls in a row, the second smaller than the first, so the second
reads nothing the first left in the shared scratch array."""

import ctypes
import math

import pytest
import torch

from causal_sliding_window_amd import inputs, swattn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc(g, W, scale):
    B, H, D = g["q"].shape
    Tmax = g["k_cache"].shape[1]
    o = torch.full_like(g["q"], float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = swattn._ptr
    rc = swattn.lib().swattn_decode_noalloc(P(g["q"]), P(g["k_cache"]), P(g["v_cache"]),
                                            P(g["seqlens"]), P(o), P(lse), B, H, D, Tmax, W,
                                            scale, stream)
    assert rc == 0, swattn.status_string(rc)
    return o, lse


def _case(name_or_shape, W):
    if name_or_shape == "decode":
        d = inputs.config_inputs("decode")
    else:
        B, H, D, Tmax, lens = name_or_shape
        d = inputs.decode_inputs(B, H, D, Tmax, "bf16", seed=3, lengths=lens)
    return {n: t.to(DEV) for n, t in d.items()}, W


def test_noalloc_decode_equals_decode_on_two_calls():
    scale = 1 / math.sqrt(128)
    # the decode workload (32 sequences, H12, 4096-row caches: 6.3 MB of partials), then
    # a smaller call (3 sequences, H2, 300-row caches, window 100)
    for g, W in (_case("decode", -1), _case((3, 2, 128, 300, [1, 177, 300]), 100)):
        o1, l1 = _noalloc(g, W, scale)
        o2, l2 = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    g, _ = _case((2, 2, 128, 64, [5, 64]), -1)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = swattn._ptr
    o = torch.empty_like(g["q"])
    # 2 x 2 heads, 2^21 cache rows in chunks of 128: 16384 partials of 129 floats > 16 MiB
    rc = swattn.lib().swattn_decode_noalloc(P(g["q"]), P(g["k_cache"]), P(g["v_cache"]),
                                            P(g["seqlens"]), P(o), None, 2, 2, 128, 1 << 21,
                                            -1, 0.1, stream)
    assert swattn.status_string(rc) == "SWATTN_ERR_TOO_LARGE"
