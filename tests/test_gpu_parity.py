"""GPU parity: libswattn (through the C ABI) against the fp64 oracle, same seeded inputs.

Bars: float32 max-abs <= 1e-5 on o, lse, dq, dk, dv; bf16 max-abs <= 2e-2 and
relative L2 <= 5e-3 on o, dq, dk, dv, and max-abs <= 1e-3 on lse.  The oracle is fed
the exact rounded inputs upcast to float64.  Full-size workloads run exactly as the
benchmark launches them and are compared on sampled heads (each head is independent).
"""

import math

import numpy as np
import pytest
import torch

from causal_sliding_window_amd import inputs, swattn
from oracle import attention as orc
from parity import (COMPOSED_ROUNDING_MISSES, EDGE_D, EDGE_T, EDGE_W, check, edge_inputs, f64,
                    only_heads, sample_heads)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(x):
    return {n: t.to(DEV) for n, t in x.items()}


def run_fwd_bwd(g, window, scale):
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], window, scale)
    dq, dk, dv = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, window, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def oracle_fwd_bwd(x, window, scale, heads=None):
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    o, lse = orc.attn_fwd(a["q"], a["k"], a["v"], window, scale, heads)
    dq, dk, dv = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], window, scale, heads)
    return o, lse, dq, dk, dv


def run_entry_points(x, window, scale):
    """Forward vs oracle, and the backward entry point fed the oracle's own forward
    output (rounded to the input dtype) and LSE, against the oracle's gradient with
    delta taken from that same output.  Isolates each kernel from the other's rounding."""
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    g = _gpu(x)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], window, scale)
    ro, rl = orc.attn_fwd(a["q"], a["k"], a["v"], window, scale)
    o_in = torch.from_numpy(ro).to(x["q"].dtype)
    lse_in = torch.from_numpy(rl).to(torch.float32)
    dq, dk, dv = swattn.bwd(g["q"], g["k"], g["v"], o_in.to(DEV), g["do"], lse_in.to(DEV),
                            window, scale)
    torch.cuda.synchronize()
    rdq, rdk, rdv = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], window, scale,
                                 o=inputs.to_f64(o_in))
    return (o, lse, dq, dk, dv), (ro, rl, rdq, rdk, rdv)


def compare_all(got, ref, dtype, heads=None, tag=""):
    names = ("o", "lse", "dq", "dk", "dv")
    for n, g, r in zip(names, got, ref):
        ga = f64(g)
        if heads is not None:
            ga = only_heads(ga, heads, "bht" if n == "lse" else "bthd")
        check(f"{tag}{n}", ga, r, dtype, lse=(n == "lse"))


# ----------------------------------------------------------------------------- fp32
def test_tiny_config_fp32():
    """B1 H2 T128 D64, fp32, full causal, seed 0: every output against the oracle."""
    x = inputs.config_inputs("tiny")
    scale = 1 / math.sqrt(64)
    compare_all(run_fwd_bwd(_gpu(x), -1, scale), oracle_fwd_bwd(x, -1, scale), torch.float32)


@pytest.mark.parametrize("T", [1, 33, 130, 257])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [-1, 1, 17, 64])
def test_fp32_shapes(T, D, W):
    x = inputs.training_inputs(2, T, 2, D, "f32", seed=T + D + W)
    scale = 1 / math.sqrt(D)
    compare_all(run_fwd_bwd(_gpu(x), W, scale), oracle_fwd_bwd(x, W, scale), torch.float32)
    compare_all(*run_entry_points(x, W, scale), torch.float32)


# ----------------------------------------------------------------------------- bf16, small shapes
@pytest.mark.parametrize("T", EDGE_T)
@pytest.mark.parametrize("D", EDGE_D)
@pytest.mark.parametrize("W", EDGE_W)
def test_bf16_shapes(T, D, W):
    """Ragged lengths and window edges mid-tile, inputs drawn like the training workloads;
    each stage in isolation (the backward gets the oracle's o and LSE)."""
    x = edge_inputs(inputs, T, W, D)
    scale = 1 / math.sqrt(D)
    compare_all(*run_entry_points(x, W, scale), torch.bfloat16)


@pytest.mark.parametrize("T", EDGE_T)
@pytest.mark.parametrize("D", EDGE_D)
@pytest.mark.parametrize("W", EDGE_W)
def test_bf16_shapes_composed(T, D, W):
    """The same sweep composed as a training step runs it: GPU forward, then the GPU
    backward fed that forward's o and LSE, every output against the exact gradient of
    the exact forward.  Cases where rounding o to bf16 alone already puts the oracle's
    own gradient outside the bar (derived on the CPU in tests/test_rounding_floor.py)
    are skipped."""
    if (T, W, D) in COMPOSED_ROUNDING_MISSES:
        pytest.skip("rounding o to bf16 alone moves the exact gradient outside the bar "
                    "(tests/test_rounding_floor.py)")
    x = edge_inputs(inputs, T, W, D)
    scale = 1 / math.sqrt(D)
    compare_all(run_fwd_bwd(_gpu(x), W, scale), oracle_fwd_bwd(x, W, scale), torch.bfloat16,
                tag=f"T{T} W{W} D{D} ")


def test_bf16_raw_normal_qk():
    """Un-normalised N(0,1) Q and K: larger logits than the QK-normed workloads."""
    x = inputs.training_inputs(2, 700, 2, 128, "bf16", seed=11, qk_norm=False)
    scale = 1 / math.sqrt(128)
    for W in (-1, 512):
        compare_all(*run_entry_points(x, W, scale), torch.bfloat16)


def test_bf16_attention_sink():
    """Every query puts most of its weight on key 0 (q = q + 6u, k[0] = 20u for a unit
    u; dO scaled by 0.05 so that |dV| stays below 4): the tiles of key 0 hold P of
    0.25 to 1 far from the diagonal, so the dK/dV pass takes its hi + lo path for P
    there and the single-bf16 path elsewhere in the same launch.

    Only the stage-isolated comparison is made (the backward gets the oracle's o and
    LSE).  On this input dP - delta cancels to a few percent of dP for every query,
    so the bf16 rounding of the forward's o (through delta = dO . o) moves dq by
    ~2% relative L2 against the exact gradient, whatever the kernels do."""
    x = inputs.training_inputs(1, 512, 2, 128, "bf16", seed=23, qk_norm=True)
    u = torch.randn(128, generator=torch.Generator().manual_seed(5), dtype=torch.float64)
    u = (u / u.norm()).to(torch.float32)
    q = x["q"].float() + 6.0 * u
    k = x["k"].float()
    k[:, 0] = 20.0 * u
    x = {"q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": x["v"],
         "do": (x["do"].float() * 0.05).to(torch.bfloat16)}
    scale = 1 / math.sqrt(128)
    qa, ka = inputs.to_f64(x["q"]), inputs.to_f64(x["k"])
    for hh in range(2):  # large P on key 0, also far from the diagonal
        p, _ = orc.head_probs(qa[0, :, hh], ka[0, :, hh], -1, scale)
        assert p[32:, 0].min() > 0.1
    compare_all(*run_entry_points(x, -1, scale), torch.bfloat16)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [511, 512, 513, 1000])
def test_window_around_the_short_window_forms(W, D):
    """Windows up to 512 keys (and shorter than T) take the short-window kernel forms
    (two-wave forward workgroups, two key groups per dK/dV workgroup); 513 and 1000 take
    the four-wave / four-group forms with a band edge inside the sequence.  Forward
    then backward on the forward's own o and LSE, against the exact gradient."""
    x = inputs.training_inputs(1, 1100, 2, D, "bf16", seed=W + D, qk_norm=True)
    scale = 1 / math.sqrt(D)
    compare_all(run_fwd_bwd(_gpu(x), W, scale), oracle_fwd_bwd(x, W, scale), torch.bfloat16,
                tag=f"W{W} D{D} ")


def test_long_sequence_sampled():
    """T = 8192, one head, full causal and a 512 window (largest shape tested)."""
    x = inputs.training_inputs(1, 8192, 1, 128, "bf16", seed=3, qk_norm=True)
    scale = 1 / math.sqrt(128)
    g = _gpu(x)
    for W in (-1, 512):
        compare_all(run_fwd_bwd(g, W, scale), oracle_fwd_bwd(x, W, scale), torch.bfloat16)


# ----------------------------------------------------------------------------- full workloads
@pytest.mark.parametrize("name", ["small", "wide-sw"])
def test_full_config_all_heads(name):
    """The workload exactly as benchmarked: GPU forward then GPU backward, every head
    against the oracle's exact gradient."""
    c = inputs.CONFIGS[name]
    x = inputs.config_inputs(name)
    scale = 1 / math.sqrt(c["D"])
    W = c["windows"][0]
    got = run_fwd_bwd(_gpu(x), W, scale)
    compare_all(got, oracle_fwd_bwd(x, W, scale), torch.bfloat16, None, f"{name} ")


def test_mid_alt_layer_schedule_all_heads():
    """Four layers, windows 512/2048/512/2048: forwards 0..3 then backwards 3..0 on one stream."""
    c = inputs.CONFIGS["mid-alt"]
    scale = 1 / math.sqrt(c["D"])
    xs = [inputs.config_inputs("mid-alt", layer) for layer in range(4)]
    gs = [_gpu(x) for x in xs]
    fw = [swattn.fwd(g["q"], g["k"], g["v"], W, scale) for g, W in zip(gs, c["windows"])]
    bw = [None] * 4
    for layer in (3, 2, 1, 0):
        g, (o, lse) = gs[layer], fw[layer]
        bw[layer] = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, c["windows"][layer], scale)
    torch.cuda.synchronize()
    for layer in range(4):
        ref = oracle_fwd_bwd(xs[layer], c["windows"][layer], scale)
        compare_all(fw[layer] + bw[layer], ref, torch.bfloat16, None, f"layer{layer} ")


# ----------------------------------------------------------------------------- decode
def test_sssl_layer_schedule_sampled():
    """The "SSSL" pattern (windows 512, 512, 512, 2048) at the mid model's shape: forwards
    0..3 then backwards 3..0 on one stream, as the benchmark runs it; every layer
    compared on sampled heads."""
    c = inputs.CONFIGS["sssl"]
    scale = 1 / math.sqrt(c["D"])
    xs = [inputs.config_inputs("sssl", layer) for layer in range(4)]
    gs = [_gpu(x) for x in xs]
    fw = [swattn.fwd(g["q"], g["k"], g["v"], c["windows"][i], scale) for i, g in enumerate(gs)]
    bw = [None] * 4
    for layer in (3, 2, 1, 0):
        g, (o, lse) = gs[layer], fw[layer]
        bw[layer] = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, c["windows"][layer], scale)
    torch.cuda.synchronize()
    heads = sample_heads(c["B"], c["H"], 3, seed=11)
    for layer in range(4):
        ref = oracle_fwd_bwd(xs[layer], c["windows"][layer], scale, heads)
        compare_all(fw[layer] + bw[layer], ref, torch.bfloat16, heads, f"layer{layer} ")


def _decode_oracle(d, W, scale):
    a = {n: inputs.to_f64(d[n]) for n in ("q", "k_cache", "v_cache")}
    return orc.attn_decode(a["q"], a["k_cache"], a["v_cache"], d["seqlens"].numpy(), W, scale)


@pytest.mark.parametrize("W", [-1, 1024])
def test_decode_config(W):
    """32 sequences, H12 D128 bf16, lengths 512..4096 (seed 7): every sequence and head."""
    d = inputs.config_inputs("decode")
    g = _gpu(d)
    scale = 1 / math.sqrt(128)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    check("decode o", o, ro, torch.bfloat16)
    check("decode lse", lse, rl, torch.bfloat16, lse=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [-1, 1, 100, 256, 257, 300])
def test_decode_shapes(dtype, D, W):
    """Lengths and windows on and next to the edges of the split kernel's 256-row
    chunks (one, two and three chunks per sequence)."""
    lens = [1, 2, 255, 256, 257, 511, 512, 513, 700, 700]
    d = inputs.decode_inputs(len(lens), 3, D, 700, dtype, seed=D + W, lengths=lens)
    g = _gpu(d)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    td = inputs.DTYPES[dtype]
    check("o", o, ro, td)
    check("lse", lse, rl, td, lse=True)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
@pytest.mark.parametrize("W,Tmax", [(-1, 1024), (1024, 1500), (300, 1100), (1, 600)])
def test_decode_many_heads_short_ranges(dtype, D, W, Tmax):
    """24 x 12 = 288 (b, h) pairs, more than one per compute unit, with visible ranges of
    at most 1024 rows (one to four 256-row chunks): lengths on and next to the chunk
    edges, an empty sequence, and lengths past the window."""
    base = [0, 1, 2, 255, 256, 257, 511, 512, 513, 767, 768, 769, 1023, 1024, 1025, 1100,
            1300, 1499, 1500, 40, 600, 700, 900, 1000]
    lens = [min(x, Tmax) for x in base]
    d = inputs.decode_inputs(len(lens), 12, D, Tmax, dtype, seed=D + W + Tmax, lengths=lens)
    g = _gpu(d)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    td = inputs.DTYPES[dtype]
    assert torch.all(o[0] == 0) and torch.all(lse[0] == -math.inf)  # the empty sequence
    check("o", o, ro, td)
    check("lse", lse[1:], rl[1:], td, lse=True)


@pytest.mark.parametrize("Hkv", [None, 4, 2])
@pytest.mark.parametrize("W", [-1, 300])
def test_decode_ignores_workspace_contents(Hkv, W):
    """The workspace is filled with NaN before the call: only the partials of chunks
    with visible rows are read by the merge, and sequences whose range is one chunk
    (or empty) are written by the split kernels directly.  Ungrouped (256-row chunks),
    grouped on the matrix cores (groups of 3) and on the vector ALU (groups of 6 at
    D = 64)."""
    lens = [0, 1, 2, 100, 255, 256, 257, 700, 1200, 1500]
    D = 64 if Hkv == 2 else 128
    H = 12
    d = inputs.decode_inputs(len(lens), H, D, 1500, "bf16", seed=31 + (Hkv or 0), lengths=lens,
                             Hkv=Hkv)
    g = _gpu(d)
    scale = 1 / math.sqrt(D)
    nbytes = swattn.swattn_decode_workspace_size(len(lens), H, D, 1500, W)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale,
                           workspace=ws)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    assert torch.all(o[0] == 0) and torch.all(lse[0] == -math.inf)  # the empty sequence
    check("o", o, ro, torch.bfloat16)
    check("lse", lse[1:], rl[1:], torch.bfloat16, lse=True)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("W", [-1, 9000])
def test_decode_long_cache(dtype, D, W):
    """Caches of 20000 rows: up to 79 chunks of 256 rows per sequence, so the merge
    runs several batches of chunks per thread (D = 128: 32 chunks per batch; D = 64:
    64)."""
    lens = [20000, 9001, 4097]
    d = inputs.decode_inputs(len(lens), 2, D, 20000, dtype, seed=11, lengths=lens)
    g = _gpu(d)
    scale = 1 / math.sqrt(D)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], W, scale)
    torch.cuda.synchronize()
    ro, rl = _decode_oracle(d, W, scale)
    td = inputs.DTYPES[dtype]
    check("o", o, ro, td)
    check("lse", lse, rl, td, lse=True)


def test_decode_clamps_and_empty():
    """seqlens above Tmax is clamped to Tmax; seqlens 0 gives o = 0, lse = -inf."""
    d = inputs.decode_inputs(3, 2, 128, 300, "bf16", seed=1, lengths=[0, 300, 300])
    g = _gpu(d)
    for n in ("q", "k_cache", "v_cache"):
        g[n][2] = g[n][1]  # sequences 1 and 2 hold the same data
    g["seqlens"] = torch.tensor([0, 5000, 300], dtype=torch.int32, device=DEV)
    o, lse = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], -1, 0.1)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.equal(o[1], o[2]) and torch.equal(lse[1], lse[2])


def test_decode_never_reads_past_length():
    lens = [5, 300, 1000]
    d = inputs.decode_inputs(3, 4, 128, 1024, "bf16", seed=2, lengths=lens)
    g = _gpu(d)
    o1, l1 = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], -1, 0.09)
    for b, L in enumerate(lens):
        g["k_cache"][b, L:] = float("nan")
        g["v_cache"][b, L:] = float("nan")
    o2, l2 = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], -1, 0.09)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_invariant_to_cache_padding():
    d = inputs.decode_inputs(2, 2, 128, 600, "bf16", seed=4, lengths=[600, 333])
    g = _gpu(d)
    o1, l1 = swattn.decode(g["q"], g["k_cache"], g["v_cache"], g["seqlens"], 256, 0.1)
    big_k = torch.zeros(2, 2000, 2, 128, dtype=torch.bfloat16, device=DEV)
    big_v = torch.zeros_like(big_k)
    big_k[:, :600], big_v[:, :600] = g["k_cache"], g["v_cache"]
    o2, l2 = swattn.decode(g["q"], big_k.contiguous(), big_v.contiguous(), g["seqlens"], 256, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("W", [-1, 200])
def test_decode_matches_forward_last_row(W):
    """Decode of the token at position L-1 equals forward row L-1 on the same prefix."""
    T, H, D = 777, 4, 128
    x = inputs.training_inputs(1, T, H, D, "bf16", seed=9, qk_norm=True)
    g = _gpu(x)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], W, 1 / math.sqrt(D))
    q_last = g["q"][:, T - 1].contiguous()
    od, ld = swattn.decode(q_last, g["k"], g["v"], torch.tensor([T], dtype=torch.int32, device=DEV),
                           W, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    assert (od.float() - o[:, T - 1].float()).abs().max().item() <= 2e-2
    assert (ld - lse[:, :, T - 1]).abs().max().item() <= 1e-4


# ----------------------------------------------------------------------------- properties
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_ge_T_bitwise_equals_full_causal(dtype):
    T = 300
    x = inputs.training_inputs(2, T, 2, 128, dtype, seed=1, qk_norm=True)
    g = _gpu(x)
    full = run_fwd_bwd(g, -1, 0.1)
    for W in (T, T + 5, 1 << 20):
        for a, b in zip(run_fwd_bwd(g, W, 0.1), full):
            assert torch.equal(a, b)


def test_repeat_calls_bitwise_deterministic():
    x = inputs.training_inputs(2, 1000, 3, 128, "bf16", seed=8, qk_norm=True)
    g = _gpu(x)
    r1 = run_fwd_bwd(g, 333, 0.09)
    r2 = run_fwd_bwd(g, 333, 0.09)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    x = inputs.training_inputs(1, 200, 2, 64, "bf16", seed=2, qk_norm=True)
    g = _gpu(x)
    ref = run_fwd_bwd(g, 50, 0.125)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = swattn.fwd(g["q"], g["k"], g["v"], 50, 0.125)
        grads = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, 50, 0.125)
    s.synchronize()
    for a, b in zip((o, lse) + grads, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_stages(dtype):
    """swattn_bwd is exactly swattn_bwd_dq then swattn_bwd_dkdv on one workspace
    (bitwise); the dQ pass leaves delta = rowsum(dO * o) in the workspace, equal to
    the preprocess's up to summation order; dK/dV fed the preprocess's delta agrees."""
    D = 64 if dtype == "f32" else 128
    x = inputs.training_inputs(2, 300, 3, D, dtype, seed=5, qk_norm=True)
    g = _gpu(x)
    W, sc = 100, 1.0 / math.sqrt(D)
    o, lse = swattn.fwd(g["q"], g["k"], g["v"], W, sc)
    ref = swattn.bwd(g["q"], g["k"], g["v"], o, g["do"], lse, W, sc)
    B, T, H, _ = g["q"].shape
    ws = torch.zeros(swattn.swattn_bwd_workspace_size(B, H, T, D), dtype=torch.uint8, device=DEV)
    dq, dk, dv = (torch.empty_like(g["q"]) for _ in range(3))
    swattn.swattn_bwd_dq(g["q"], g["k"], g["v"], o, g["do"], lse, ws, dq, W, sc)
    swattn.swattn_bwd_dkdv(g["q"], g["k"], g["v"], g["do"], lse, ws, dk, dv, W, sc)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)
    delta_dq = ws.view(torch.float32)[: B * H * T].clone()
    ws2 = torch.zeros_like(ws)
    swattn.swattn_bwd_preprocess(o, g["do"], ws2)
    dk2, dv2 = torch.empty_like(dk), torch.empty_like(dv)
    swattn.swattn_bwd_dkdv(g["q"], g["k"], g["v"], g["do"], lse, ws2, dk2, dv2, W, sc)
    torch.cuda.synchronize()
    delta_pre = ws2.view(torch.float32)[: B * H * T]
    ref_delta = (o.double() * g["do"].double()).sum(-1).permute(0, 2, 1).reshape(-1)
    tol = 1e-4 * (1 + ref_delta.abs())
    assert torch.all((delta_dq.double() - ref_delta).abs() <= tol)
    assert torch.all((delta_pre.double() - ref_delta).abs() <= tol)
    bar = 1e-5 if dtype == "f32" else 2e-2
    assert (dk2.double() - dk.double()).abs().max().item() <= bar
    assert (dv2.double() - dv.double()).abs().max().item() <= bar


def test_w1_gradients_vanish():
    """W = 1: o = v and dv = dO after bf16 rounding; dq and dk vanish."""
    x = inputs.training_inputs(1, 130, 2, 128, "bf16", seed=5, qk_norm=True)
    o, lse, dq, dk, dv = run_fwd_bwd(_gpu(x), 1, 0.1)
    assert torch.equal(o.cpu(), x["v"])
    assert torch.equal(dv.cpu(), x["do"])
    # dS = P (dP - delta) vanishes up to fp32 rounding (dP and delta are summed in different orders)
    assert dq.abs().max().item() <= 1e-4 and dk.abs().max().item() <= 1e-4
