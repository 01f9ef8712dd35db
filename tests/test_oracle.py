"""Pins of the fp64 oracle against things other than itself.

Nothing on the nanochat pages prints attention values, so the oracle is pinned by
a hand-derived closed form (tests/golden), special cases with closed forms
(T=1, W=1, equal logits), invariants (row sums, shift invariance, gradient
identities), brute force in pure-Python loops, an independent library routine
(PyTorch CPU scaled_dot_product_attention in float64 with autograd) and central
finite differences.  Each pin is chosen so that a dropped term, a wrong sign or
index, an off-by-one window edge or a transposed operand fails at least one.
"""

import json
import math
import os
import re

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _expr(s):
    s = re.sub(r"ln(\d+)", lambda m: repr(math.log(int(m.group(1)))), s)
    return float(eval(s, {"__builtins__": {}}, {}))  # fixture text written by hand in this repo


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _expr(x) if isinstance(x, str) else float(x)


def _rand(*shape):
    return RNG.standard_normal(shape)


# ----------------------------------------------------------------------------- golden
def test_golden_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_t3.json")))
    q, k, v, do = _arr(g["q"]), _arr(g["k_expr"]), _arr(g["v"]), _arr(g["do"])
    o, lse = orc.head_fwd(q, k, v, -1, g["scale"])
    np.testing.assert_allclose(o, _arr(g["full"]["o"]), atol=1e-14)
    np.testing.assert_allclose(lse, _arr(g["full"]["lse"]), atol=1e-14)
    dq, dk, dv = orc.head_bwd(q, k, v, do, -1, g["scale"])
    np.testing.assert_allclose(dq, _arr(g["full"]["dq"]), atol=1e-14)
    np.testing.assert_allclose(dk, _arr(g["full"]["dk"]), atol=1e-14)
    np.testing.assert_allclose(dv, _arr(g["full"]["dv"]), atol=1e-14)
    o2, lse2 = orc.head_fwd(q, k, v, 2, g["scale"])
    np.testing.assert_allclose(o2, _arr(g["window2"]["o"]), atol=1e-14)
    np.testing.assert_allclose(lse2, _arr(g["window2"]["lse"]), atol=1e-14)


# ----------------------------------------------------------------------------- masks
def test_visible_mask_definition():
    vis = orc.visible_mask(6, 6, 3)
    for i in range(6):
        for j in range(6):
            assert vis[i, j] == (j <= i and i - j < 3)
    assert orc.visible_mask(5, 5, -1).sum() == 15
    with pytest.raises(ValueError):
        orc.visible_mask(4, 4, 0)


# ----------------------------------------------------------------------------- forward
GRID = [(T, W, D) for T in (1, 2, 3, 5, 8, 17, 128) for W in (1, 2, 3, -1, "T-1", "T", "T+5")
        for D in (4, 8, 64) if not (T > 17 and D == 4)]


def _w(W, T):
    if isinstance(W, str):
        W = eval(W, {"__builtins__": {}}, {"T": T})
        return W if W >= 1 else -1
    return W


@pytest.mark.parametrize("T,W,D", GRID)
def test_rows_sum_to_one(T, W, D):
    W = _w(W, T)
    q, k = _rand(T, D), _rand(T, D)
    p, lse = orc.head_probs(q, k, W, 1 / math.sqrt(D))
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)
    assert np.all(p[~orc.visible_mask(T, T, W)] == 0)
    assert np.all(np.isfinite(lse))


def test_T1_identity():
    q, k, v, do = _rand(1, 8), _rand(1, 8), _rand(1, 8), _rand(1, 8)
    o, lse = orc.head_fwd(q, k, v, -1, 0.3)
    np.testing.assert_array_equal(o, v)
    assert lse[0] == pytest.approx(0.3 * float(q[0] @ k[0]), abs=1e-15)
    dq, dk, dv = orc.head_bwd(q, k, v, do, -1, 0.3)
    np.testing.assert_allclose(dq, 0, atol=1e-15)
    np.testing.assert_allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv, do, atol=1e-15)


@pytest.mark.parametrize("T", [2, 7, 33])
def test_window_one_is_identity(T):
    """W = 1 pins the window reading: a query sees exactly itself."""
    D = 8
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    o, lse = orc.head_fwd(q, k, v, 1, 0.5)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("td,td->t", q, k), atol=1e-14)
    dq, dk, dv = orc.head_bwd(q, k, v, do, 1, 0.5)
    np.testing.assert_allclose(dq, 0, atol=1e-14)
    np.testing.assert_allclose(dk, 0, atol=1e-14)
    np.testing.assert_allclose(dv, do, atol=1e-14)


@pytest.mark.parametrize("T", [3, 16, 50])
def test_window_two_counts_two_keys(T):
    """W = 2: each row i >= 1 is a two-way softmax over keys i-1 and i."""
    D = 4
    q, k, v = _rand(T, D), _rand(T, D), _rand(T, D)
    o, _ = orc.head_fwd(q, k, v, 2, 1.0)
    for i in range(1, T):
        a, b = float(q[i] @ k[i - 1]), float(q[i] @ k[i])
        w = 1.0 / (1.0 + math.exp(b - a))
        np.testing.assert_allclose(o[i], w * v[i - 1] + (1 - w) * v[i], atol=1e-13)


@pytest.mark.parametrize("T", [1, 5, 64])
def test_window_ge_T_equals_full_causal(T):
    D = 8
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    o_full, l_full = orc.head_fwd(q, k, v, -1, 0.7)
    for W in (T, T + 5):
        o, l = orc.head_fwd(q, k, v, W, 0.7)
        np.testing.assert_array_equal(o, o_full)
        np.testing.assert_array_equal(l, l_full)
        for a, b in zip(orc.head_bwd(q, k, v, do, W, 0.7), orc.head_bwd(q, k, v, do, -1, 0.7)):
            np.testing.assert_array_equal(a, b)
    if T > 1:  # W = T-1 drops key 0 for the last row
        o, _ = orc.head_fwd(q, k, v, T - 1, 0.7)
        assert not np.allclose(o[-1], o_full[-1])


@pytest.mark.parametrize("T,W", [(9, -1), (9, 3), (40, 7), (40, 40)])
def test_equal_logits_give_window_mean(T, W):
    """Q = 0 (or all K rows equal): o_i is the mean of v over the n_i band keys."""
    D = 6
    v = _rand(T, D)
    n = np.array([min(i + 1, W) if W > 0 else i + 1 for i in range(T)])
    mean = np.array([v[i - n[i] + 1:i + 1].mean(axis=0) for i in range(T)])
    o, lse = orc.head_fwd(np.zeros((T, D)), _rand(T, D), v, W, 0.9)
    np.testing.assert_allclose(o, mean, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(n), atol=1e-14)
    q = _rand(T, D)
    krow = _rand(1, D)
    o, lse = orc.head_fwd(q, np.repeat(krow, T, axis=0), v, W, 0.9)
    np.testing.assert_allclose(o, mean, atol=1e-13)
    np.testing.assert_allclose(lse, 0.9 * (q @ krow[0]) + np.log(n), atol=1e-13)


@pytest.mark.parametrize("W", [-1, 4])
def test_key_shift_invariance(W):
    T, D = 20, 8
    q, k, v = _rand(T, D), _rand(T, D), _rand(T, D)
    c = _rand(D)
    o1, l1 = orc.head_fwd(q, k, v, W, 0.4)
    o2, l2 = orc.head_fwd(q, k + c[None, :], v, W, 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, 0.4 * (q @ c), atol=1e-12)


def test_last_row_is_textbook_softmax():
    from scipy.special import softmax, logsumexp
    T, D = 31, 16
    q, k, v = _rand(T, D), _rand(T, D), _rand(T, D)
    s = 0.25 * (k @ q[-1])
    o, lse = orc.head_fwd(q, k, v, -1, 0.25)
    np.testing.assert_allclose(o[-1], softmax(s) @ v, atol=1e-14)
    assert lse[-1] == pytest.approx(logsumexp(s), abs=1e-13)


# ----------------------------------------------------------------------------- brute force
def _brute(q, k, v, do, W, scale, o_given=None):
    """Pure-Python loops, straight from the scalar definition (delta from o_given if set)."""
    T, D = len(q), len(q[0])
    vis = [[j <= i and (W < 0 or i - j < W) for j in range(T)] for i in range(T)]
    s = [[scale * sum(q[i][d] * k[j][d] for d in range(D)) for j in range(T)] for i in range(T)]
    lse = []
    p = [[0.0] * T for _ in range(T)]
    for i in range(T):
        m = max(s[i][j] for j in range(T) if vis[i][j])
        tot = sum(math.exp(s[i][j] - m) for j in range(T) if vis[i][j])
        lse.append(m + math.log(tot))
        for j in range(T):
            if vis[i][j]:
                p[i][j] = math.exp(s[i][j] - lse[i])
    o = [[sum(p[i][j] * v[j][d] for j in range(T)) for d in range(D)] for i in range(T)]
    dv = [[sum(p[i][j] * do[i][d] for i in range(T)) for d in range(D)] for j in range(T)]
    ob = o if o_given is None else o_given
    delta = [sum(do[i][d] * ob[i][d] for d in range(D)) for i in range(T)]
    ds = [[p[i][j] * (sum(do[i][d] * v[j][d] for d in range(D)) - delta[i]) for j in range(T)]
          for i in range(T)]
    dq = [[scale * sum(ds[i][j] * k[j][d] for j in range(T)) for d in range(D)] for i in range(T)]
    dk = [[scale * sum(ds[i][j] * q[i][d] for i in range(T)) for d in range(D)] for j in range(T)]
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("T,W,D", [(1, -1, 3), (4, -1, 3), (6, 2, 5), (7, 3, 2), (9, 9, 4), (8, 1, 3)])
def test_brute_force_loops(T, W, D):
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    o_b, l_b, dq_b, dk_b, dv_b = _brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), W, 0.6)
    o, lse = orc.head_fwd(q, k, v, W, 0.6)
    dq, dk, dv = orc.head_bwd(q, k, v, do, W, 0.6)
    for a, b in [(o, o_b), (lse, l_b), (dq, dq_b), (dk, dk_b), (dv, dv_b)]:
        np.testing.assert_allclose(a, np.array(b), atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("T,W,D", [(1, -1, 8), (17, -1, 8), (64, 5, 16), (130, 33, 32), (256, -1, 64), (256, 128, 64)])
def test_matches_torch_sdpa_fp64(T, W, D):
    B, H = 2, 3
    x = {n: RNG.standard_normal((B, T, H, D)) for n in ("q", "k", "v", "do")}
    scale = 1 / math.sqrt(D)
    o, lse = orc.attn_fwd(x["q"], x["k"], x["v"], W, scale)
    dq, dk, dv = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], W, scale)
    t = {n: torch.tensor(a).permute(0, 2, 1, 3).contiguous().requires_grad_(n != "do")
         for n, a in x.items()}
    band = np.tril(np.ones((T, T), bool))  # j <= i, built without the oracle
    if W > 0:
        band &= np.triu(np.ones((T, T), bool), -(W - 1))  # i - j <= W - 1
    mask = torch.tensor(band)
    ref = torch.nn.functional.scaled_dot_product_attention(t["q"], t["k"], t["v"], attn_mask=mask, scale=scale)
    ref.backward(t["do"])
    s = scale * t["q"].detach() @ t["k"].detach().transpose(-1, -2)
    ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    tr = lambda a: a.detach().permute(0, 2, 1, 3).numpy()  # noqa: E731
    np.testing.assert_allclose(o, tr(ref), atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tr(t["q"].grad), atol=1e-12)
    np.testing.assert_allclose(dk, tr(t["k"].grad), atol=1e-12)
    np.testing.assert_allclose(dv, tr(t["v"].grad), atol=1e-12)


# ----------------------------------------------------------------------------- gradients
@pytest.mark.parametrize("T,W,D", [(1, -1, 2), (4, -1, 4), (6, 2, 3), (8, 3, 8), (8, -1, 8), (5, 1, 2)])
def test_finite_differences(T, W, D):
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    scale, h = 0.8, 1e-6

    def loss(q_, k_, v_):
        return float((orc.head_fwd(q_, k_, v_, W, scale)[0] * do).sum())

    grads = orc.head_bwd(q, k, v, do, W, scale)
    for which, g in enumerate(grads):
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.abs(fd - g).max() / max(1.0, np.abs(g).max())
        assert err < 1e-6, (which, err)


@pytest.mark.parametrize("T,W", [(64, -1), (64, 9), (200, 50)])
def test_gradient_identities(T, W):
    D = 16
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    dq, dk, dv = orc.head_bwd(q, k, v, do, W, 0.3)
    np.testing.assert_allclose(dk.sum(axis=0), 0, atol=1e-12)             # softmax rows are shift invariant
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)  # p rows sum to 1
    assert float((q * dq).sum()) == pytest.approx(float((k * dk).sum()), abs=1e-11)  # Q*a, K/a invariance
    p, _ = orc.head_probs(q, k, W, 0.3)
    o = p @ v
    ds = p * (do @ v.T - (do * o).sum(1)[:, None])
    np.testing.assert_allclose(ds.sum(axis=1), 0, atol=1e-13)


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("W", [-1, 1, 5, 64])
def test_decode_is_last_row_of_forward(W):
    B, H, D, Tmax = 3, 2, 8, 40
    kc, vc = _rand(B, Tmax, H, D), _rand(B, Tmax, H, D)
    q = _rand(B, H, D)
    lens = np.array([1, 17, 40])
    kc_nan, vc_nan = kc.copy(), vc.copy()
    for b, L in enumerate(lens):
        kc_nan[b, L:] = np.nan
        vc_nan[b, L:] = np.nan
    o, lse = orc.attn_decode(q, kc_nan, vc_nan, lens, W, 0.35)
    for b, L in enumerate(lens):
        for h in range(H):
            qq = kc[b, :L, h].copy()
            qq[L - 1] = q[b, h]
            of, lf = orc.head_fwd(qq, kc[b, :L, h], vc[b, :L, h], W, 0.35)
            np.testing.assert_allclose(o[b, h], of[L - 1], atol=1e-14)
            assert lse[b, h] == pytest.approx(lf[L - 1], abs=1e-14)


def test_decode_empty_sequence():
    o, lse = orc.attn_decode(np.ones((1, 1, 4)), np.ones((1, 3, 1, 4)), np.ones((1, 3, 1, 4)),
                             np.array([0]), -1, 1.0)
    assert np.all(o == 0) and lse[0, 0] == -np.inf


def test_lse_merge_of_partition_equals_whole():
    """Split-KV identity the decode kernels rely on, checked on the oracle's own quantities."""
    L, D = 300, 8
    q, k, v = _rand(1, D), _rand(L, D), _rand(L, D)
    o_all, l_all = orc.attn_decode(q[None], k[None, :, None], v[None, :, None], np.array([L]), -1, 0.5)
    parts = [(0, 37), (37, 38), (38, 200), (200, 300)]
    os_, ls_ = [], []
    for a, b in parts:
        s = 0.5 * (k[a:b] @ q[0])
        m = s.max()
        ls_.append(m + math.log(np.exp(s - m).sum()))
        os_.append(np.exp(s - ls_[-1]) @ v[a:b])
    lse = np.logaddexp.reduce(ls_)
    o = sum(math.exp(l_ - lse) * o_ for l_, o_ in zip(ls_, os_))
    assert lse == pytest.approx(l_all[0, 0], abs=1e-13)
    np.testing.assert_allclose(o, o_all[0, 0], atol=1e-13)


# ----------------------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible bugs in the oracle (on the CPU) and check a pin fails for each."""
    T, D = 6, 3
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 2, 0.6)
    good_mask = orc.visible_mask

    def off_by_one(n_q, n_k, window, q_pos0=0):  # i - j <= W instead of < W
        i = q_pos0 + np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        return (j <= i) & ((i - j) <= window) if window > 0 else (j <= i)

    monkeypatch.setattr(orc, "visible_mask", off_by_one)
    assert not np.allclose(orc.head_fwd(q, k, v, 2, 0.6)[0], np.array(ref[0]))
    monkeypatch.setattr(orc, "visible_mask", good_mask)
    np.testing.assert_allclose(orc.head_fwd(q, k, v, 2, 0.6)[0], np.array(ref[0]), atol=1e-12)
    # a transposed operand in dk (ds instead of ds^T) breaks the brute-force match
    p, _ = orc.head_probs(q, k, 2, 0.6)
    ds = p * (do @ v.T - (do * (p @ v)).sum(1)[:, None])
    assert not np.allclose(0.6 * (ds @ q), np.array(ref[3]))


@pytest.mark.parametrize("T,W,D", [(5, -1, 3), (7, 3, 4)])
def test_delta_from_given_output(T, W, D):
    """With a supplied (perturbed) forward output, delta is taken from it; with the exact
    output the result is the exact gradient."""
    q, k, v, do = _rand(T, D), _rand(T, D), _rand(T, D), _rand(T, D)
    o, _ = orc.head_fwd(q, k, v, W, 0.6)
    for a, b in zip(orc.head_bwd(q, k, v, do, W, 0.6, o=o), orc.head_bwd(q, k, v, do, W, 0.6)):
        np.testing.assert_allclose(a, b, atol=1e-14)
    o_pert = o + 1e-3 * _rand(T, D)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), W, 0.6, o_pert.tolist())
    got = orc.head_bwd(q, k, v, do, W, 0.6, o=o_pert)
    for a, b in zip(got, ref[2:]):
        np.testing.assert_allclose(a, np.array(b), atol=1e-12)
    assert not np.allclose(got[0], orc.head_bwd(q, k, v, do, W, 0.6)[0], atol=1e-9)


# ----------------------------------------------------------------------------- grouped K/V heads
@pytest.mark.parametrize("H,Hkv", [(6, 1), (6, 2), (6, 3), (4, 4)])
@pytest.mark.parametrize("T,W", [(17, -1), (40, 5)])
def test_gqa_matches_torch_sdpa_enable_gqa(H, Hkv, T, W):
    """Grouped-query forward and backward against PyTorch's CPU SDPA in fp64 with
    enable_gqa (its own head mapping, query head h on K/V head h // (H / Hkv)) and
    autograd: a wrong group mapping (h % Hkv) or a missing sum over a group fails."""
    B, D = 2, 8
    x = {n: RNG.standard_normal((B, T, H if n in ("q", "do") else Hkv, D))
         for n in ("q", "k", "v", "do")}
    scale = 1 / math.sqrt(D)
    o, lse = orc.attn_fwd(x["q"], x["k"], x["v"], W, scale)
    dq, dk, dv = orc.attn_bwd(x["q"], x["k"], x["v"], x["do"], W, scale)
    assert dk.shape == (B, T, Hkv, D) and dv.shape == (B, T, Hkv, D)
    t = {n: torch.tensor(a).permute(0, 2, 1, 3).contiguous().requires_grad_(n != "do")
         for n, a in x.items()}
    band = np.tril(np.ones((T, T), bool))
    if W > 0:
        band &= np.triu(np.ones((T, T), bool), -(W - 1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        t["q"], t["k"], t["v"], attn_mask=torch.tensor(band), scale=scale, enable_gqa=True)
    ref.backward(t["do"])
    tr = lambda a: a.detach().permute(0, 2, 1, 3).numpy()  # noqa: E731
    np.testing.assert_allclose(o, tr(ref), atol=1e-12)
    np.testing.assert_allclose(dq, tr(t["q"].grad), atol=1e-12)
    np.testing.assert_allclose(dk, tr(t["k"].grad), atol=1e-12)
    np.testing.assert_allclose(dv, tr(t["v"].grad), atol=1e-12)
    # lse of each query head against the logsumexp of its own K/V head's logits
    kv = np.repeat(x["k"], H // Hkv, axis=2)
    s = scale * np.einsum("bihd,bjhd->bhij", x["q"], kv)
    s = np.where(band, s, -np.inf)
    m = s.max(-1, keepdims=True)
    np.testing.assert_allclose(lse, (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0],
                               atol=1e-12)


def test_gqa_finite_differences():
    """dk and dv of a shared K/V head are the derivatives of L = sum dO . o over all the
    query heads that read it (central differences, one K/V head shared by three)."""
    B, T, H, Hkv, D, W = 1, 5, 3, 1, 3, 3
    q, do = _rand(B, T, H, D), _rand(B, T, H, D)
    k, v = _rand(B, T, Hkv, D), _rand(B, T, Hkv, D)
    scale, h = 0.7, 1e-6

    def loss(k_, v_):
        return float((orc.attn_fwd(q, k_, v_, W, scale)[0] * do).sum())

    _, dk, dv = orc.attn_bwd(q, k, v, do, W, scale)
    for which, g in ((0, dk), (1, dv)):
        fd = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            args_p, args_m = [k.copy(), v.copy()], [k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(fd - g).max() / max(1.0, np.abs(g).max()) < 1e-6, which


@pytest.mark.parametrize("W", [-1, 3])
def test_gqa_decode_is_last_row_of_forward(W):
    """Grouped decode reads K/V head h // (H / Hkv), like the grouped forward."""
    B, T, H, Hkv, D = 2, 9, 4, 2, 5
    q, k, v = _rand(B, T, H, D), _rand(B, T, Hkv, D), _rand(B, T, Hkv, D)
    o, lse = orc.attn_fwd(q, k, v, W, 0.5)
    od, ld = orc.attn_decode(q[:, T - 1], k, v, np.array([T, T]), W, 0.5)
    np.testing.assert_allclose(od, o[:, T - 1], atol=1e-14)
    np.testing.assert_allclose(ld, lse[:, :, T - 1], atol=1e-14)


def test_gqa_rejects_uneven_groups():
    q, k = _rand(1, 4, 6, 2), _rand(1, 4, 4, 2)
    with pytest.raises(ValueError):
        orc.attn_fwd(q, k, k, -1, 1.0)


# ----------------------------------------------------------------------------- prefill
def _prefill_case(B=2, Tq=5, H=4, Hkv=2, D=6, Tmax=20):
    return (_rand(B, Tq, H, D), _rand(B, Tq, Hkv, D), _rand(B, Tq, Hkv, D),
            _rand(B, Tmax, Hkv, D), _rand(B, Tmax, Hkv, D))


@pytest.mark.parametrize("W", [-1, 1, 3, 8])
def test_prefill_on_empty_cache_is_the_forward(W):
    q, kn, vn, kc, vc = _prefill_case()
    o, lse, kc2, vc2 = orc.attn_prefill(q, kn, vn, kc, vc, [0, 0], W, 0.4)
    fo, fl = orc.attn_fwd(q, kn, vn, W, 0.4)
    np.testing.assert_allclose(o, fo, atol=1e-13)
    np.testing.assert_allclose(lse, fl, atol=1e-13)
    np.testing.assert_array_equal(kc2[:, :5], kn)
    np.testing.assert_array_equal(kc2[:, 5:], kc[:, 5:])  # rows past the chunk untouched


@pytest.mark.parametrize("W", [-1, 4])
def test_prefill_in_two_chunks_is_the_forward_of_the_whole(W):
    """Chunk 1 at an empty cache, then chunk 2 at seqlens = len(chunk 1): the second
    chunk's outputs are the last rows of the forward over both chunks."""
    B, H, Hkv, D, Tmax = 2, 4, 2, 6, 16
    q = _rand(B, 9, H, D)
    k, v = _rand(B, 9, Hkv, D), _rand(B, 9, Hkv, D)
    kc, vc = np.zeros((B, Tmax, Hkv, D)), np.zeros((B, Tmax, Hkv, D))
    _, _, kc, vc = orc.attn_prefill(q[:, :4], k[:, :4], v[:, :4], kc, vc, [0, 0], W, 0.5)
    o2, l2, _, _ = orc.attn_prefill(q[:, 4:], k[:, 4:], v[:, 4:], kc, vc, [4, 4], W, 0.5)
    fo, fl = orc.attn_fwd(q, k, v, W, 0.5)
    np.testing.assert_allclose(o2, fo[:, 4:], atol=1e-13)
    np.testing.assert_allclose(l2, fl[:, :, 4:], atol=1e-13)


@pytest.mark.parametrize("W", [-1, 2, 6])
def test_prefill_last_row_is_decode_on_the_updated_cache(W):
    q, kn, vn, kc, vc = _prefill_case()
    seq = np.array([3, 11])
    o, lse, kc2, vc2 = orc.attn_prefill(q, kn, vn, kc, vc, seq, W, 0.7)
    od, ld = orc.attn_decode(q[:, -1], kc2, vc2, seq + 5, W, 0.7)
    np.testing.assert_allclose(o[:, -1], od, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, -1], ld, atol=1e-13)


def test_prefill_matches_torch_sdpa_offset_mask():
    """An independent routine: SDPA (fp64) over the updated cache with the offset causal
    and window mask built here, K/V heads repeated per group."""
    q, kn, vn, kc, vc = _prefill_case(Tq=6, Tmax=24)
    W, scale, seq = 5, 0.6, [7, 2]
    o, lse, kc2, vc2 = orc.attn_prefill(q, kn, vn, kc, vc, seq, W, scale)
    for b, L0 in enumerate(seq):
        n = L0 + 6
        i = np.arange(6)[:, None] + L0
        j = np.arange(n)[None, :]
        mask = torch.tensor((j <= i) & (i - j < W))
        t = lambda a: torch.tensor(a).permute(1, 0, 2)  # noqa: E731  [T, h, D] -> [h, T, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            t(q[b]), t(kc2[b, :n]), t(vc2[b, :n]), attn_mask=mask, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(o[b], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_prefill_clamps_seqlens_to_the_cache():
    q, kn, vn, kc, vc = _prefill_case(Tmax=12)
    o, lse, kc2, _ = orc.attn_prefill(q, kn, vn, kc, vc, [30, -3], -1, 0.5)
    o7, l7, kc7, _ = orc.attn_prefill(q, kn, vn, kc, vc, [7, 0], -1, 0.5)  # 12 - 5 = 7
    np.testing.assert_array_equal(o, o7)
    np.testing.assert_array_equal(kc2, kc7)
    np.testing.assert_array_equal(kc2[0, 7:12], kn[0])
