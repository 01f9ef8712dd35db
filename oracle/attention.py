"""Plain fp64 definition of causal sliding-window attention (forward, backward, decode).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never by the product path.

Sources (the nanochat pages):

* nanochat guide ("Train your own ChatGPT", apidog), section 5 "Flash Attention
  unification": the model's attention is one call taking q, k, v with causal
  masking and a ``window_size`` argument; off Hopper the same call falls back to
  PyTorch's scaled-dot-product attention, i.e. the result is plain masked
  softmax(scale * Q K^T) V.
* same guide, section 1 "GPT model", feature list: sliding-window attention with a
  per-layer pattern that alternates short and long context (e.g. "SSSL").
* time-to-GPT-2 post (Jan-29 leaderboard), list of the biggest wins: the Flash
  Attention 3 kernels allow the ``window_size`` argument for alternating patterns.
* same guide, section 6 "Inference engine": the KV cache is filled and read
  through the kernels' with-KV-cache entry; decode is one new query token per
  sequence against that cache.

Readings where the pages are silent:

* ``window = W >= 1``: query i sees key j iff ``j <= i`` and ``i - j < W``, i.e. the
  W most recent keys including itself.  ``window < 0`` means full causal.
  ``window == 0`` is rejected.
* LSE is the natural log of the softmax denominator, ``LSE_i = m_i + ln l_i``.
* Backward is the analytic gradient of ``L = sum_i dO_i . o_i`` with respect to
  q, k, v (LSE is an output only; nothing flows back through it).
* Decode: ``seqlens[b] = L`` counts valid cache rows including the new token; the
  query sits at position ``L - 1``.  ``L == 0`` gives o = 0, LSE = -inf.
* Prefill with cache append (same section 6: the engine fills the cache through the
  kernels' with-KV-cache entry; one chunk of Tq new tokens at a time): with
  ``L0 = seqlens[b]`` rows already cached, the chunk's K/V rows are written at rows
  ``L0 .. L0 + Tq - 1`` and query i sits at position ``L0 + i``.  ``seqlens`` is
  clamped to ``[0, Tmax - Tq]`` so that every written row exists (the reading for
  a length the pages leave unbounded).
* Grouped-query attention (same guide, section 1 feature list: fewer K/V heads than
  query heads, for faster inference; the multi-query case, one K/V head, is in the
  architecture list of the release article).  The pages do not say which query
  heads share a K/V head; the reading here is contiguous groups: with H query heads
  and Hkv K/V heads (H a multiple of Hkv), query head h uses K/V head h // (H / Hkv).
  Its gradients with respect to k and v are the sums over the group's query heads.

Every array is float64.  No blocking, fusion or reordering: each function is the
definition, written out with NumPy matrix products as its only library steps.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask",
    "head_probs",
    "head_fwd",
    "head_bwd",
    "attn_fwd",
    "attn_bwd",
    "attn_decode",
    "attn_prefill",
]


def _check_window(window: int) -> int:
    window = int(window)
    if window == 0:
        raise ValueError("window must be >= 1, or negative for full causal")
    return window


def visible_mask(n_q: int, n_k: int, window: int, q_pos0: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k]: may the query at position ``q_pos0 + i`` attend to key ``j``?

    Causal masking from the guide's section 5 (causal flag on); the window from
    section 1's sliding-window feature.  Visible iff ``j <= i`` and, when a window
    ``W >= 1`` is given, ``i - j < W``.
    """
    window = _check_window(window)
    i = q_pos0 + np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = j <= i
    if window > 0:
        vis = vis & ((i - j) < window)
    return vis


def head_probs(q: np.ndarray, k: np.ndarray, window: int, scale: float,
               q_pos0: int = 0):
    """Softmax probabilities and LSE of one head.

    q: [n_q, D], k: [n_k, D].  Returns (p [n_q, n_k], lse [n_q]) with
    ``s = scale * q k^T``, ``m_i = max over visible j``, ``l_i = sum over visible of
    exp(s_ij - m_i)``, ``LSE_i = m_i + ln l_i`` and ``p_ij = exp(s_ij - LSE_i)`` on
    visible entries, 0 elsewhere.  A row with no visible key gets LSE = -inf and
    an all-zero p row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vis = visible_mask(q.shape[0], k.shape[0], window, q_pos0)
    s = scale * (q @ k.T)
    s_vis = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s_vis.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s_vis - m[:, None]), 0.0)
    ell = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, m + np.log(ell), -np.inf)
    p = np.where(vis, np.exp(s - np.where(any_vis, lse, 0.0)[:, None]), 0.0)
    return p, lse


def head_fwd(q, k, v, window: int, scale: float):
    """Forward of one head: q, k, v [T, D] -> (o [T, D], lse [T]); ``o = p v``."""
    p, lse = head_probs(q, k, window, scale)
    o = p @ np.asarray(v, dtype=np.float64)
    return o, lse


def head_bwd(q, k, v, do, window: int, scale: float, o=None):
    """Analytic gradients of ``L = sum_i dO_i . o_i`` for one head.

    With p from :func:`head_probs` and o = p v:
      dv = p^T dO;  dp = dO v^T;  delta_i = dO_i . o_i;
      ds = p * (dp - delta);  dq = scale * ds k;  dk = scale * ds^T q.
    Returns (dq, dk, dv), each [T, D].

    ``o``: optional forward output to take delta from (the backward entry point
    receives the stored forward output and forms delta from it); by default the
    exact o = p v is used, which gives the exact gradient.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    p, _ = head_probs(q, k, window, scale)
    o = p @ v if o is None else np.asarray(o, dtype=np.float64)
    dv = p.T @ do
    dp = do @ v.T
    delta = (do * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _group(H: int, k) -> int:
    """Query heads per K/V head (1 without grouping), from k's head count."""
    Hkv = np.shape(k)[2]
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"{H} query heads cannot be grouped over {Hkv} K/V heads")
    return H // Hkv


def _heads(B: int, H: int, heads):
    if heads is None:
        return [(b, h) for b in range(B) for h in range(H)]
    return [(int(b), int(h)) for b, h in heads]


def attn_fwd(q, k, v, window: int, scale: float, heads=None):
    """Forward over q [B, T, H, D] and k, v [B, T, Hkv, D] (Hkv = H, or a divisor
    of H for grouped-query attention: query head h reads K/V head h // (H / Hkv)).

    Returns (o [B, T, H, D], lse [B, H, T]).  With ``heads`` (a list of (b, h))
    only those heads are computed; the others are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, T, H, D = q.shape
    G = _group(H, k)
    o = np.full((B, T, H, D), np.nan)
    lse = np.full((B, H, T), np.nan)
    for b, h in _heads(B, H, heads):
        o[b, :, h, :], lse[b, h, :] = head_fwd(q[b, :, h, :], k[b, :, h // G, :],
                                               v[b, :, h // G, :], window, scale)
    return o, lse


def attn_bwd(q, k, v, do, window: int, scale: float, heads=None, o=None):
    """Backward over q, do [B, T, H, D] and k, v [B, T, Hkv, D] -> (dq [B, T, H, D],
    dk, dv [B, T, Hkv, D]); see :func:`head_bwd` (``o``, optional [B, T, H, D]: the
    forward output delta is taken from).  A K/V head's dk and dv sum the gradients of
    every query head that reads it; with ``heads``, the sum runs over the listed ones
    and K/V heads no listed head reads are left NaN."""
    q = np.asarray(q, dtype=np.float64)
    B, T, H, D = q.shape
    G = _group(H, k)
    dq = np.full((B, T, H, D), np.nan)
    dk = np.full((B, T, H // G, D), np.nan)
    dv = np.full((B, T, H // G, D), np.nan)
    for b, h in _heads(B, H, heads):
        dq[b, :, h, :], gk, gv = head_bwd(
            q[b, :, h, :], k[b, :, h // G, :], v[b, :, h // G, :], do[b, :, h, :],
            window, scale, None if o is None else o[b, :, h, :])
        if np.isnan(dk[b, 0, h // G, 0]):
            dk[b, :, h // G, :] = 0.0
            dv[b, :, h // G, :] = 0.0
        dk[b, :, h // G, :] += gk
        dv[b, :, h // G, :] += gv
    return dq, dk, dv


def attn_decode(q, k_cache, v_cache, seqlens, window: int, scale: float,
                seqs=None):
    """One-token decode against a KV cache (guide section 6, "Inference engine").

    q: [B, H, D]; k_cache, v_cache: [B, Tmax, Hkv, D] (query head h reads K/V head
    h // (H / Hkv)); seqlens: [B] ints.
    Sequence b's query sits at position ``L = seqlens[b]`` minus one and sees the
    cache rows ``0 .. L-1`` that pass :func:`visible_mask`.  Rows ``>= L`` are
    never read.  Returns (o [B, H, D], lse [B, H]); with ``seqs`` only those
    sequences are computed (others NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, D = q.shape
    G = _group(H, k_cache)
    Tmax = k_cache.shape[1]
    o = np.full((B, H, D), np.nan)
    lse = np.full((B, H), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seqlens[b])
        if L < 0 or L > Tmax:
            raise ValueError(f"seqlens[{b}] = {L} outside [0, {Tmax}]")
        for h in range(H):
            if L == 0:
                o[b, h] = 0.0
                lse[b, h] = -np.inf
                continue
            kb = np.asarray(k_cache[b, :L, h // G, :], dtype=np.float64)
            vb = np.asarray(v_cache[b, :L, h // G, :], dtype=np.float64)
            p, l_ = head_probs(q[b, h][None, :], kb, window, scale, q_pos0=L - 1)
            o[b, h] = (p @ vb)[0]
            lse[b, h] = l_[0]
    return o, lse


def attn_prefill(q, k_new, v_new, k_cache, v_cache, seqlens, window: int, scale: float):
    """Chunked prefill against a KV cache, appending the chunk's K/V first.

    q: [B, Tq, H, D]; k_new, v_new: [B, Tq, Hkv, D]; k_cache, v_cache: [B, Tmax, Hkv, D];
    seqlens: [B] ints, the cache rows already filled.  For sequence b, with
    L0 = min(max(seqlens[b], 0), Tmax - Tq), rows L0 .. L0 + Tq - 1 of copies of the
    caches receive k_new[b], v_new[b]; query i then attends, as position L0 + i, to
    the rows of the updated cache that :func:`visible_mask` allows (rows past
    L0 + i are never visible).  Returns (o [B, Tq, H, D], lse [B, H, Tq], k_cache',
    v_cache').
    """
    q = np.asarray(q, dtype=np.float64)
    B, Tq, H, D = q.shape
    G = _group(H, k_cache)
    Tmax = k_cache.shape[1]
    if Tq > Tmax:
        raise ValueError(f"a chunk of {Tq} rows does not fit a cache of {Tmax}")
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    o = np.zeros((B, Tq, H, D))
    lse = np.zeros((B, H, Tq))
    for b in range(B):
        L0 = min(max(int(seqlens[b]), 0), Tmax - Tq)
        kc[b, L0:L0 + Tq] = k_new[b]
        vc[b, L0:L0 + Tq] = v_new[b]
        for h in range(H):
            kb, vb = kc[b, :L0 + Tq, h // G, :], vc[b, :L0 + Tq, h // G, :]
            p, lse[b, h] = head_probs(q[b, :, h, :], kb, window, scale, q_pos0=L0)
            o[b, :, h, :] = p @ vb
    return o, lse, kc, vc
