"""GPU parity of the grouped-query entry points (*_gqa) against the fp64 oracle.

H query heads share Hkv K/V heads in contiguous groups (query head h reads K/V head
h // (H / Hkv)); dk and dv of a K/V head sum over its group.  Bars as in the other GPU
tests (bf16 max-abs <= 2e-2 and relative L2 <= 5e-3 on o, dq; max-abs <= 1e-3 on
lse), except that dk and dv, sums over up to H / Hkv heads, reach magnitudes where the
bf16 rounding of the output alone passes 2e-2 (half an ulp is 0.031 at |x| = 9.8):
there the max-abs bar holds elementwise on top of that rounding, |err| <= 2e-2 +
2^-9 |ref|, with the same relative-L2 bar.
"""

import math

import pytest
import torch

from causal_sliding_window_amd import inputs, swattn
from oracle import attention as orc
from parity import check, f64, only_heads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(x):
    return {n: t.to(DEV) for n, t in x.items()}


def _isolated(x, window, scale):
    """Forward against the oracle, and the backward fed the oracle's forward output
    (rounded to bf16) and LSE against the oracle's gradient with delta from that
    output: each kernel stage is compared without the other's rounding."""
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    g = _gpu(x)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], window, scale)
    ro, rl = orc.attn_fwd(a["q"], a["k"], a["v"], window, scale)
    o_in = torch.from_numpy(ro).to(torch.bfloat16)
    lse_in = torch.from_numpy(rl).to(torch.float32)
    dq, dk, dv = swattn.bwd(g["q"], g["k"], g["v"], o_in.to(DEV), g["do"], lse_in.to(DEV),
                            window, scale)
    torch.cuda.synchronize()
    rdq, rdk, rdv = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], window, scale,
                                 o=inputs.to_f64(o_in))
    for n, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk),
                        ("dv", dv, rdv)):
        check(n, got, ref, torch.bfloat16, lse=(n == "lse"), out_ulp=n in ("dk", "dv"))


@pytest.mark.parametrize("H,Hkv", [(6, 1), (6, 2), (6, 3), (8, 2)])
@pytest.mark.parametrize("T,W,D", [(129, -1, 128), (300, 65, 128), (64, 1, 64), (257, 200, 64)])
def test_gqa_stages_vs_oracle(H, Hkv, T, W, D):
    x = inputs.training_inputs(2, T, H, D, "bf16", seed=H * 10 + Hkv + T, qk_norm=True, Hkv=Hkv)
    _isolated(x, W, 1 / math.sqrt(D))


@pytest.mark.parametrize("W", [-1, 100])
def test_gqa_full_path_vs_oracle(W):
    """Forward then backward on the forward's own o and lse, against the exact gradient."""
    B, T, H, Hkv, D = 2, 384, 6, 2, 128
    x = inputs.training_inputs(B, T, H, D, "bf16", seed=3, qk_norm=True, Hkv=Hkv)
    g = _gpu(x)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], W, scale)
    dq, dk, dv = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, W, scale)
    torch.cuda.synchronize()
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    ro, rl = orc.attn_fwd(a["q"], a["k"], a["v"], W, scale)
    rdq, rdk, rdv = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], W, scale)
    for n, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rdq), ("dk", dk, rdk),
                        ("dv", dv, rdv)):
        check(n, got, ref, torch.bfloat16, lse=(n == "lse"), out_ulp=n in ("dk", "dv"))


def test_gqa_equals_ungrouped_on_repeated_kv():
    """With each K/V head repeated over its group, the ungrouped entry points compute the
    same thing: o, lse and dq bitwise (same kernels, same operands), and dk, dv equal to
    the sums over each group of the ungrouped per-head gradients."""
    B, T, H, Hkv, D, W = 2, 200, 6, 2, 128, 77
    x = _gpu(inputs.training_inputs(B, T, H, D, "bf16", seed=5, qk_norm=True, Hkv=Hkv))
    scale = 1 / math.sqrt(D)
    G = H // Hkv
    rep = {n: x[n].repeat_interleave(G, dim=2).contiguous() for n in ("k", "v")}
    o, lse = swattn.fwd(x["q"], x["k"], x["v"], W, scale)
    o2, lse2 = swattn.fwd(x["q"], rep["k"], rep["v"], W, scale)
    dq, dk, dv = swattn.bwd(x["q"], x["k"], x["v"], o, x["do"], lse, W, scale)
    dq2, dk2, dv2 = swattn.bwd(x["q"], rep["k"], rep["v"], o2, x["do"], lse2, W, scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)
    # the reference sums G per-head gradients that were each rounded to bf16 (up to half
    # an ulp each): it carries roundings of its own, so only the rounding-aware bar applies
    for got, per_head in ((dk, dk2), (dv, dv2)):
        ref = f64(per_head).reshape(B, T, Hkv, G, D).sum(axis=3)
        check("group sum", got, ref, torch.bfloat16, out_ulp=True, exact_ref=False)


def test_gqa_full_size_sampled():
    """The small training workload's shape (B8 T2048 D128, RMS-normalised q, k) with six
    query heads on two K/V heads, as the grouped entry points run it at full size;
    compared on two K/V heads (and their six query heads)."""
    B, T, H, Hkv, D = 8, 2048, 6, 2, 128
    x = inputs.training_inputs(B, T, H, D, "bf16", seed=0, qk_norm=True, Hkv=Hkv)
    g = _gpu(x)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], -1, scale)
    dq, dk, dv = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, -1, scale)
    torch.cuda.synchronize()
    kv_heads = [(0, 0), (B - 1, Hkv - 1)]
    heads = [(b, hk * (H // Hkv) + j) for b, hk in kv_heads for j in range(H // Hkv)]
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    ro, rl = orc.attn_fwd(a["q"], a["k"], a["v"], -1, scale, heads)
    rdq, rdk, rdv = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], -1, scale, heads)
    check("o", only_heads(f64(o), heads), ro, torch.bfloat16)
    check("lse", only_heads(f64(lse), heads, "bht"), rl, torch.bfloat16, lse=True)
    check("dq", only_heads(f64(dq), heads), rdq, torch.bfloat16)
    check("dk", only_heads(f64(dk), kv_heads), rdk, torch.bfloat16, out_ulp=True)
    check("dv", only_heads(f64(dv), kv_heads), rdv, torch.bfloat16, out_ulp=True)


def _decode_oracle(d, W, scale):
    a = {n: inputs.to_f64(d[n]) for n in ("q", "k_cache", "v_cache")}
    return orc.attn_decode(a["q"], a["k_cache"], a["v_cache"], d["seqlens"].numpy(), W, scale)


@pytest.mark.parametrize("H,Hkv", [(8, 1), (8, 2), (8, 4), (12, 3), (64, 2), (40, 1)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [-1, 100])
def test_gqa_decode_vs_oracle(H, Hkv, D, W):
    """Groups of 2 to 40 query heads (the bf16 D = 128 kernel takes them 32 at a time:
    40 needs two batches, 32 fills one); lengths of 0, 1, one row past a chunk, and
    ragged chunk tails."""
    lens = [0, 1, 129, 700, 1000, 257]
    d = inputs.decode_inputs(len(lens), H, D, 1000, "bf16", seed=H + Hkv + D, lengths=lens,
                             Hkv=Hkv)
    g = _gpu(d)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    check("o", o, ro, torch.bfloat16)
    # sequence 0 is empty: o = 0 (checked above) and lse = -inf
    assert torch.all(lse[0] == -math.inf)
    check("lse", lse[1:], rl[1:], torch.bfloat16, lse=True)


@pytest.mark.parametrize("D", [64, 128])
def test_gqa_decode_equals_ungrouped_on_repeated_cache(D):
    """Grouped decode reads each cache row once for its group; with the cache repeated
    over the group, the ungrouped decode computes the same thing.  The two agree to
    the bf16 bar and each meets it against the oracle: the grouped kernels take
    128-row chunks where the ungrouped one takes 256 (D = 64: vector ALU both), and at
    D = 128 the grouped matrix-core kernel rounds P to bf16 before P V as the forward
    does."""
    B, H, Hkv, Tmax = 6, 12, 4, 3000
    d = inputs.decode_inputs(B, H, D, Tmax, "bf16", seed=9, Hkv=Hkv)
    g = _gpu(d)
    G = H // Hkv
    kc = g["k_cache"].repeat_interleave(G, dim=2).contiguous()
    vc = g["v_cache"].repeat_interleave(G, dim=2).contiguous()
    for W in (-1, 512):
        o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W)
        o2, lse2 = swattn.decode(g["q"], kc, vc, g["seqlens"], W)
        torch.cuda.synchronize()
        ro, rl = _decode_oracle(d, W, 1 / math.sqrt(D))
        for got in (o, o2):
            check("o", got, ro, torch.bfloat16)
        for got in (lse, lse2):
            check("lse", got, rl, torch.bfloat16, lse=True)
        check("o vs ungrouped", o, f64(o2), torch.bfloat16)
        check("lse vs ungrouped", lse, f64(lse2), torch.bfloat16, lse=True)


@pytest.mark.parametrize("H,Hkv", [(12, 6), (12, 4), (16, 1), (33, 1)])
@pytest.mark.parametrize("W", [-1, 127, 128, 129, 5000])
def test_gqa_decode_chunk_edges(H, Hkv, W):
    """Lengths on and next to the 128-row chunk edges (127, 128, 129, 256, 384 + 1) and
    windows either side of one chunk; groups of 2, 3, 16 and 33 query heads (the last
    with a one-head second batch on the matrix-core kernel)."""
    lens = [127, 128, 129, 256, 385, 1024]
    d = inputs.decode_inputs(len(lens), H, 128, 1024, "bf16", seed=H + W, lengths=lens, Hkv=Hkv)
    g = _gpu(d)
    scale = 1 / math.sqrt(128)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    check("o", o, ro, torch.bfloat16)
    check("lse", lse, rl, torch.bfloat16, lse=True)


_EDGES = [0, 1, 2, 127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 512, 513, 767, 768, 769,
          1023, 1024, 1025, 2047, 2048, 3000, 4095, 4096]


@pytest.mark.parametrize("B,H,Hkv,Tmax,W", [(32, 24, 8, 1024, -1), (32, 12, 4, 4096, -1),
                                            (32, 24, 12, 2048, -1),
                                            (32, 64, 2, 4096, -1), (128, 24, 8, 512, 129),
                                            (128, 24, 8, 512, 300), (64, 12, 4, 2048, 1000)])
def test_gqa_decode_large_grids(B, H, Hkv, Tmax, W):
    """Grids of 1024 and more workgroups on the matrix-core kernel (B Hkv ceil(visible /
    256) >= 1024): groups of 2, 3, 12 and 32 heads, up to 128 sequences; lengths on and next
    to the 128- and 256-row edges, an empty sequence, lengths past the window."""
    lens = [0] + [min(_EDGES[1 + i % (len(_EDGES) - 1)], Tmax) for i in range(B - 1)]
    d = inputs.decode_inputs(B, H, 128, Tmax, "bf16", seed=B + H + W, lengths=lens, Hkv=Hkv)
    g = _gpu(d)
    scale = 1 / math.sqrt(128)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    check("o", o, ro, torch.bfloat16)
    assert torch.all(o[0] == 0) and torch.all(lse[0] == -math.inf)  # the empty sequence
    check("lse", lse[1:], rl[1:], torch.bfloat16, lse=True)


def test_gqa_decode_long_cache_mqa():
    """One K/V head for all query heads (multi-query), 20000-row caches."""
    lens = [20000, 9001]
    d = inputs.decode_inputs(2, 8, 128, 20000, "bf16", seed=4, lengths=lens, Hkv=1)
    g = _gpu(d)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], -1)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, -1, 1 / math.sqrt(128))
    check("o", o, ro, torch.bfloat16)
    check("lse", lse, rl, torch.bfloat16, lse=True)


def test_gqa_rejects_uneven_groups():
    x = _gpu(inputs.training_inputs(1, 16, 6, 64, "bf16", seed=1, Hkv=4))
    with pytest.raises(swattn.SwattnError):
        swattn.fwd(x["q"], x["k"], x["v"])
