"""GPU parity of attention with the QK-norm + rotary prologue fused into the passes
(swattn_fwd_rope, swattn_bwd_rope, and their _gqa forms with K/V head groups) against
the oracle composed from its prologue and attention.

The composed reference, stage by stage: q' (written by the fused forward) and k' (the
keys-only prologue) against the fp64 oracle prologue; o and LSE against the oracle
attention on those bf16 q', k' and v; dq, dk against the oracle prologue's backward
(on the raw q, k) applied to the oracle attention's exact gradients with respect to
q', k'; dv against the oracle attention's.  The GPU runs a training
step the fused way: the keys-only prologue, then swattn_fwd_rope (which also writes q'),
then swattn_bwd_rope on that forward's o and LSE.  Bars: the bf16 bars.  dq and dk are
the attention's gradients of q', k' mapped back through the QK norm, whose backward
multiplies a gradient by 1 / rms of the raw vector (the raw rms is 0.5 .. 4 here, so up
to 2): the attention stage keeps its 2e-2 max-abs bar before that map, i.e. dq and dk are
held to |err| <= 2e-2 max(1, 1 / rms) + 2^-9 |ref| (the last term the output's own bf16
rounding), with the same relative-L2 bar.
"""

import math

import numpy as np
import pytest
import torch

from causal_sliding_window_amd import inputs, swattn
from oracle import attention as orc
from oracle import prologue as pro
from parity import check, f64, only_heads, sample_heads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _raw(B, T, H, D, seed, Hkv=None):
    """Raw projections: N(0, 1) scaled per vector by 0.5 .. 4, so the norm has work to do;
    v and dO N(0, 1).  k and v have Hkv heads (H by default)."""
    Hkv = H if Hkv is None else Hkv
    x = inputs.training_inputs(B, T, H, D, "bf16", seed=seed, qk_norm=False, Hkv=Hkv)
    g = torch.Generator().manual_seed(seed + 99)
    sq = 0.5 + 3.5 * torch.rand((B, T, H, 1), generator=g)
    sk = 0.5 + 3.5 * torch.rand((B, T, Hkv, 1), generator=g)
    return {"q": (x["q"].float() * sq).to(torch.bfloat16),
            "k": (x["k"].float() * sk).to(torch.bfloat16), "v": x["v"], "do": x["do"]}


def _bf16(a):
    return inputs.to_f64(torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16))


def _reference(x, W, scale, pos0, base, eps, qp, kp, heads=None):
    """The oracle on the GPU's own transformed q' and k' (bf16, checked separately against
    the oracle prologue): a bf16 rounding of q' or k' that lands on the other neighbour
    than the rounded exact value moves a logit by up to ~1e-3, the whole LSE bar, so
    each stage is compared on the same inputs."""
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    o, lse = orc.attn_fwd(qp, kp, a["v"], W, scale, heads)
    dqp, dkp, dv = orc.attn_bwd(qp, kp, a["v"], a["do"], W, scale, heads)
    dq = pro.qk_norm_rope_bwd(a["q"], np.nan_to_num(dqp), pos0, base, eps)
    dk = pro.qk_norm_rope_bwd(a["k"], np.nan_to_num(dkp), pos0, base, eps)
    if heads is not None:  # heads outside the sample: NaN (not compared)
        dq = only_heads(dq, heads)
        dk = only_heads(dk, heads)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _fused_step(x, W, scale, pos_off, base, eps, grouped=False):
    """One training step the fused way; ``grouped`` takes the _gqa entry points (k, v
    with their own head count)."""
    g = {n: t.to(DEV) for n, t in x.items()}
    B, T, H, D = g["q"].shape
    Hkv = g["k"].shape[2]
    k_rope, q_rope = torch.empty_like(g["k"]), torch.empty_like(g["q"])
    o, dq = torch.empty_like(g["q"]), torch.empty_like(g["q"])
    dk, dv = torch.empty_like(g["k"]), torch.empty_like(g["k"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    po = None if pos_off is None else torch.tensor(pos_off, dtype=torch.int32, device=DEV)
    swattn.swattn_qk_norm_rope(None, g["k"], None, k_rope, po, base, eps)  # keys only
    if grouped:
        ws = torch.empty(swattn.swattn_bwd_gqa_workspace_size(B, H, Hkv, T, D),
                         dtype=torch.uint8, device=DEV)
        swattn.swattn_fwd_rope_gqa(g["q"], k_rope, g["v"], o, lse, q_rope, W, scale, po, base,
                                   eps)
        swattn.swattn_bwd_rope_gqa(g["q"], g["k"], q_rope, k_rope, g["v"], o, g["do"], lse, dq,
                                   dk, dv, W, scale, ws, po, base, eps)
    else:
        ws = torch.empty(swattn.swattn_bwd_workspace_size(B, H, T, D), dtype=torch.uint8,
                         device=DEV)
        swattn.swattn_fwd_rope(g["q"], k_rope, g["v"], o, lse, q_rope, W, scale, po, base, eps)
        swattn.swattn_bwd_rope(g["q"], g["k"], q_rope, k_rope, g["v"], o, g["do"], lse, dq, dk,
                               dv, W, scale, ws, po, base, eps)
    torch.cuda.synchronize()
    return {"q'": q_rope, "k'": k_rope, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _check_prologue_outputs(got, x, pos0, base, eps, tag=""):
    """q' (written by the fused forward) and k' (the keys-only prologue) against the
    oracle prologue; returns them as float64 for the attention reference."""
    qp, kp = inputs.to_f64(got["q'"]), inputs.to_f64(got["k'"])
    check(f"{tag}q'", qp, pro.qk_norm_rope(inputs.to_f64(x["q"]), pos0, base, eps), torch.bfloat16)
    check(f"{tag}k'", kp, pro.qk_norm_rope(inputs.to_f64(x["k"]), pos0, base, eps), torch.bfloat16)
    return qp, kp


def _norm_gain(x, eps):
    """max(1, 1 / rms) per raw head vector [B, T, H, 1]: the largest factor by which the
    QK norm's backward scales the gradient it is given."""
    a = inputs.to_f64(x)
    return np.maximum(1.0, 1.0 / np.sqrt((a * a).mean(-1, keepdims=True) + eps))


def _compare(got, ref, heads=None, tag="", grouped=False, x=None, eps=1e-6):
    """dq, dk with the gain of the norm's backward (from the raw ``x``); dv of a grouped
    step sums over the group's query heads (magnitudes up to ~10): it takes the
    rounding-aware bar as dq and dk do."""
    scaled = ("dq", "dk", "dv") if grouped else ("dq", "dk")
    gains = {"dq": _norm_gain(x["q"], eps), "dk": _norm_gain(x["k"], eps)}
    for n in ("o", "lse", "dq", "dk", "dv"):
        g = f64(got[n])
        if heads is not None:
            g = only_heads(g, heads, "bht" if n == "lse" else "bthd")
        check(f"{tag}{n}", g, ref[n], torch.bfloat16, lse=(n == "lse"), out_ulp=n in scaled,
              gain=gains.get(n))


@pytest.mark.parametrize("T,D,W", [(300, 128, 100), (129, 64, -1), (520, 128, -1),
                                   (257, 64, 65)])
@pytest.mark.parametrize("pos_off,base,eps", [(None, 1e4, 1e-6), ([0, 37], 1e4, 1e-6),
                                              ([-5, 4000], 5e5, 0.25)])
def test_fused_prologue_attention_step(T, D, W, pos_off, base, eps):
    x = _raw(2, T, 3, D, seed=T + D + W)
    scale = 1 / math.sqrt(D)
    got = _fused_step(x, W, scale, pos_off, base, eps)
    qp, kp = _check_prologue_outputs(got, x, pos_off, base, eps, f"T{T} D{D} W{W} ")
    ref = _reference(x, W, scale, pos_off, base, eps, qp, kp)
    _compare(got, ref, tag=f"T{T} D{D} W{W} ", x=x, eps=eps)


def test_fused_prologue_small_workload_sampled():
    """The small workload's shape (B8 H6 T2048 D128, full causal) with raw projections,
    compared on sampled heads."""
    c = inputs.CONFIGS["small"]
    x = _raw(c["B"], c["T"], c["H"], c["D"], seed=3)
    scale = 1 / math.sqrt(c["D"])
    got = _fused_step(x, -1, scale, None, 1e4, 1e-6)
    qp, kp = _check_prologue_outputs(got, x, None, 1e4, 1e-6, "small ")
    heads = sample_heads(c["B"], c["H"], 3, seed=2)
    ref = _reference(x, -1, scale, None, 1e4, 1e-6, qp, kp, heads)
    _compare(got, ref, heads, tag="small ", x=x)


def test_fused_equals_unfused_path():
    """The fused step against the unfused one (two-sided prologue, swattn_fwd, swattn_bwd,
    prologue backward): the same results up to rounding, and q' / k' of the fused path
    within one bf16 rounding step of the standalone prologue's."""
    B, T, H, D, W = 2, 300, 3, 128, 100
    x = _raw(B, T, H, D, seed=7)
    scale = 1 / math.sqrt(D)
    got = _fused_step(x, W, scale, [3, 0], 1e4, 1e-6)
    g = {n: t.to(DEV) for n, t in x.items()}
    po = torch.tensor([3, 0], dtype=torch.int32, device=DEV)
    yq, yk = swattn.qk_norm_rope(g["q"], g["k"], po)
    o, lse = swattn.fwd(yq, yk, g["v"], W, scale)
    dyq, dyk, dv = swattn.bwd(yq, yk, g["v"], o, g["do"], lse, W, scale)
    dq, dk = swattn.qk_norm_rope_bwd(g["q"], g["k"], dyq, dyk, po)
    torch.cuda.synchronize()
    # one bf16 step of the larger of the two, with an absolute floor of 2^-20 for values
    # near zero (the fp32 arithmetic before the rounding is good to ~1e-7 absolute there)
    a, b = got["q'"].float(), yq.float()
    big = torch.clamp(torch.maximum(a.abs(), b.abs()), min=2.0 ** -126)
    step = torch.clamp(torch.exp2(torch.floor(torch.log2(big)) - 7), min=2.0 ** -20)
    bad = (a - b).abs() > step
    assert not bad.any(), (a[bad][:8].tolist(), b[bad][:8].tolist())
    for n, a, b in (("o", got["o"], o), ("lse", got["lse"], lse), ("dv", got["dv"], dv)):
        check(f"fused vs unfused {n}", a, f64(b), torch.bfloat16, lse=(n == "lse"))
    # the unfused dq, dk are bf16 outputs themselves (rounded once more than the oracle,
    # and mapped through the norm's backward as the fused ones are): only the
    # rounding-aware bar applies, with the norm's gain
    for n, a, b in (("dq", got["dq"], dq), ("dk", got["dk"], dk)):
        check(f"fused vs unfused {n}", a, f64(b), torch.bfloat16, out_ulp=True, exact_ref=False,
              gain=_norm_gain(x[n[1]], 1e-6))


@pytest.mark.parametrize("H,Hkv", [(6, 2), (4, 1), (6, 3)])
@pytest.mark.parametrize("T,D,W", [(300, 128, 100), (129, 64, -1), (257, 128, -1),
                                   (257, 64, 65)])
def test_fused_prologue_grouped_step(H, Hkv, T, D, W):
    """The _gqa forms: H query heads over Hkv K/V heads, against the composed oracle
    (its attention sums each K/V head's gradients over the group before the prologue's
    backward maps them; the library maps each query head's share first, the same up to
    rounding since the mapping is linear in dk')."""
    pos_off = [2, 301]
    x = _raw(2, T, H, D, seed=H * 7 + Hkv + T + D, Hkv=Hkv)
    scale = 1 / math.sqrt(D)
    got = _fused_step(x, W, scale, pos_off, 1e4, 1e-6, grouped=True)
    tag = f"H{H} Hkv{Hkv} T{T} D{D} W{W} "
    qp, kp = _check_prologue_outputs(got, x, pos_off, 1e4, 1e-6, tag)
    ref = _reference(x, W, scale, pos_off, 1e4, 1e-6, qp, kp)
    _compare(got, ref, tag=tag, grouped=True, x=x)


def test_fused_grouped_with_equal_heads_is_the_ungrouped_path():
    """With Hkv == H the _gqa forms launch the ungrouped kernels: identical outputs."""
    x = _raw(2, 300, 3, 128, seed=11)
    a = _fused_step(x, 100, 1 / math.sqrt(128), [0, 5], 1e4, 1e-6, grouped=True)
    b = _fused_step(x, 100, 1 / math.sqrt(128), [0, 5], 1e4, 1e-6, grouped=False)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_fused_grouped_equals_unfused_grouped_path():
    """The grouped fused step against the grouped unfused one (two-sided prologue with
    Hkv key heads, swattn_fwd_gqa, swattn_bwd_gqa, prologue backward)."""
    B, T, H, Hkv, D, W = 2, 384, 6, 2, 128, -1
    x = _raw(B, T, H, D, seed=5, Hkv=Hkv)
    scale = 1 / math.sqrt(D)
    got = _fused_step(x, W, scale, None, 1e4, 1e-6, grouped=True)
    g = {n: t.to(DEV) for n, t in x.items()}
    yq, yk = swattn.qk_norm_rope(g["q"], g["k"])
    o, lse = swattn.fwd(yq, yk, g["v"], W, scale)
    dyq, dyk, dv = swattn.bwd(yq, yk, g["v"], o, g["do"], lse, W, scale)
    dq, dk = swattn.qk_norm_rope_bwd(g["q"], g["k"], dyq, dyk)
    torch.cuda.synchronize()
    for n, a, b in (("o", got["o"], o), ("lse", got["lse"], lse), ("dv", got["dv"], dv)):
        check(f"grouped fused vs unfused {n}", a, f64(b), torch.bfloat16, lse=(n == "lse"),
              out_ulp=(n == "dv"))
    for n, a, b in (("dq", got["dq"], dq), ("dk", got["dk"], dk)):
        check(f"grouped fused vs unfused {n}", a, f64(b), torch.bfloat16, out_ulp=True,
              exact_ref=False, gain=_norm_gain(x[n[1]], 1e-6))
