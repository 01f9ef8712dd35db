"""GPU parity of the QK-norm + rotary prologue (swattn_qk_norm_rope, _bwd) against the
fp64 oracle (oracle/prologue.py).

Outputs are bf16 rounded from fp32 arithmetic (fp64 angles): the bf16 bar of the
other tests, max-abs <= 2e-2 and relative L2 <= 5e-3.  q' and k' have unit RMS, so half
an ulp of bf16 stays below 1.6e-2.  dq and dk scale with 1 / rms(x) and reach 8.6 here
(inputs with rms down to 0.5), where half an ulp is 0.031: for them the max-abs bar
holds elementwise on top of the output's own rounding, |err| <= 2e-2 + 2^-9 |ref|,
with the same relative-L2 bar.
"""

import math

import numpy as np
import pytest
import torch

from causal_sliding_window_amd import inputs, swattn
from oracle import attention as orc
from oracle import prologue as pro
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _raw(B, T, H, Hkv, D, seed):
    """Raw (un-normalised) projections: N(0, 1) scaled per vector by 0.5 .. 4, so the
    norm has work to do."""
    x = inputs.training_inputs(B, T, H, D, "bf16", seed=seed, qk_norm=False, Hkv=Hkv)
    g = torch.Generator().manual_seed(seed + 99)
    sq = 0.5 + 3.5 * torch.rand((B, T, H, 1), generator=g)
    sk = 0.5 + 3.5 * torch.rand((B, T, Hkv, 1), generator=g)
    return ((x["q"].float() * sq).to(torch.bfloat16), (x["k"].float() * sk).to(torch.bfloat16),
            x["v"])


def _f(t):
    return inputs.to_f64(t)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(6, 6), (6, 2), (4, 1)])
@pytest.mark.parametrize("offs", [None, [0, 37], [-5, 4000]])
def test_prologue_vs_oracle(D, H, Hkv, offs):
    B, T = 2, 129
    q, k, _ = _raw(B, T, H, Hkv, D, seed=D + H + Hkv)
    po = None if offs is None else torch.tensor(offs, dtype=torch.int32)
    gq, gk = q.to(DEV), k.to(DEV)
    gpo = None if po is None else po.to(DEV)
    yq, yk = swattn.qk_norm_rope(gq, gk, gpo)
    # gradients of the outputs, as the attention backward would hand them over
    dyq = torch.randn(q.shape, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    dyk = torch.randn(k.shape, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    dq, dk = swattn.qk_norm_rope_bwd(gq, gk, dyq.to(DEV), dyk.to(DEV), gpo)
    torch.cuda.synchronize()
    pos0 = None if offs is None else np.array(offs)
    check("q'", yq, pro.qk_norm_rope(_f(q), pos0), torch.bfloat16)
    check("k'", yk, pro.qk_norm_rope(_f(k), pos0), torch.bfloat16)
    check("dq", dq, pro.qk_norm_rope_bwd(_f(q), _f(dyq), pos0), torch.bfloat16, out_ulp=True)
    check("dk", dk, pro.qk_norm_rope_bwd(_f(k), _f(dyk), pos0), torch.bfloat16, out_ulp=True)


def test_prologue_base_eps_and_large_positions():
    """Another base and eps, and positions near 2^30 (fp64 angles)."""
    B, T, H, Hkv, D = 2, 33, 3, 1, 128
    q, k, _ = _raw(B, T, H, Hkv, D, seed=11)
    offs = [1 << 30, 123457]
    po = torch.tensor(offs, dtype=torch.int32, device=DEV)
    yq, yk = swattn.qk_norm_rope(q.to(DEV), k.to(DEV), po, base=500000.0, eps=0.25)
    torch.cuda.synchronize()
    check("q'", yq, pro.qk_norm_rope(_f(q), np.array(offs), 500000.0, 0.25), torch.bfloat16)
    check("k'", yk, pro.qk_norm_rope(_f(k), np.array(offs), 500000.0, 0.25), torch.bfloat16)


def test_prologue_in_place_equals_out_of_place():
    B, T, H, Hkv, D = 2, 64, 6, 2, 128
    q, k, _ = _raw(B, T, H, Hkv, D, seed=12)
    gq, gk = q.to(DEV), k.to(DEV)
    yq, yk = swattn.qk_norm_rope(gq, gk)
    dq, dk = swattn.qk_norm_rope_bwd(gq, gk, yq, yk)
    iq, ik = gq.clone(), gk.clone()
    swattn.swattn_qk_norm_rope(iq, ik, iq, ik)
    gy_q, gy_k = yq.clone(), yk.clone()
    swattn.swattn_qk_norm_rope_bwd(gq, gk, gy_q, gy_k, gy_q, gy_k)
    torch.cuda.synchronize()
    assert torch.equal(iq, yq) and torch.equal(ik, yk)
    assert torch.equal(gy_q, dq) and torch.equal(gy_k, dk)


def test_prologue_full_size():
    """The small training workload's q and k (B8 T2048 H6 D128), raw, whole tensors."""
    B, T, H, D = 8, 2048, 6, 128
    q, k, _ = _raw(B, T, H, H, D, seed=0)
    gq, gk = q.to(DEV), k.to(DEV)
    yq, yk = swattn.qk_norm_rope(gq, gk)
    dq, dk = swattn.qk_norm_rope_bwd(gq, gk, yk, yq)  # any bf16 gradients of the shapes
    torch.cuda.synchronize()
    check("q'", yq, pro.qk_norm_rope(_f(q)), torch.bfloat16)
    check("k'", yk, pro.qk_norm_rope(_f(k)), torch.bfloat16)
    check("dq", dq, pro.qk_norm_rope_bwd(_f(q), _f(yk)), torch.bfloat16, out_ulp=True)
    check("dk", dk, pro.qk_norm_rope_bwd(_f(k), _f(yq)), torch.bfloat16, out_ulp=True)


def test_prologue_then_attention():
    """Raw projections through the prologue, then the attention forward on its
    outputs: the prologue against the oracle's prologue, and the attention against the
    oracle's attention on the prologue's own bf16 outputs (each stage to its bar)."""
    B, T, H, Hkv, D, W = 2, 300, 6, 2, 128, 100
    q, k, v = _raw(B, T, H, Hkv, D, seed=13)
    yq, yk = swattn.qk_norm_rope(q.to(DEV), k.to(DEV))
    o, lse = swattn.fwd(yq, yk, v.to(DEV), W)
    torch.cuda.synchronize()
    check("q'", yq, pro.qk_norm_rope(_f(q)), torch.bfloat16)
    ro, rl = orc.attn_fwd(_f(yq), _f(yk), _f(v), W, 1 / math.sqrt(D))
    check("o", o, ro, torch.bfloat16)
    check("lse", lse, rl, torch.bfloat16, lse=True)
