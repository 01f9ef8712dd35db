"""Plain fp64 definition of the QK-norm + rotary prologue (forward and backward).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``bench.py``'s CPU leg, never
by the product path.

Sources (the nanochat pages):

* nanochat release article (followin.io), architecture list: rotary embeddings are
  the only position encoding; queries and keys are normalised (QK norm); the
  model's RMSNorm has no learnable parameters.
* nanochat guide ("Train your own ChatGPT", apidog), section 1 "GPT model",
  feature list: rotary embeddings encode relative position with no learned
  position embeddings; QK normalisation keeps large-scale training stable.

The pages name the two operations but give no formula.  Readings (the plainest
ones the rest supports):

* QK norm: per (b, t, head) D-vector, ``x_n = x / sqrt(mean_d x_d^2 + eps)``,
  no weight, applied to q and k alike.
* Rotary embedding (RoFormer's rotation): the D-vector is taken as D/2 pairs
  ``(x_i, x_{i + D/2})`` (the two halves), and pair i of the token at position p
  is rotated by the angle ``p * base^(-2i/D)``:
  ``y_i = x_i cos - x_{i+D/2} sin``, ``y_{i+D/2} = x_i sin + x_{i+D/2} cos``,
  base 10000 unless given.  The token's position is ``p = pos0_b + t`` (``pos0_b``
  the sequence's offset, 0 for a training batch).
* Order: the rotation keeps the RMS of a vector, and the norm has no weight, so
  norm-then-rotate and rotate-then-norm are the same map; the definition below
  normalises first.
* Backward: the analytic gradient of ``sum y . dy`` with respect to x.
"""

import numpy as np


def rope_angles(pos: np.ndarray, D: int, base: float = 10000.0) -> np.ndarray:
    """Angles [len(pos), D/2]: position p times base^(-2i/D) for pair i (fp64)."""
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def _positions(B: int, T: int, pos0) -> np.ndarray:
    """[B, T] token positions pos0_b + t (pos0: None, an int, or per-sequence ints;
    negative offsets count as 0)."""
    off = np.zeros(B, dtype=np.int64) if pos0 is None else np.broadcast_to(
        np.asarray(pos0, dtype=np.int64), (B,))
    return np.maximum(off, 0)[:, None] + np.arange(T)[None, :]


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean over the last axis of x^2 + eps)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rotate(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Rotate pairs (x_i, x_{i+D/2}) of x [..., D] by ang [..., D/2] (broadcast)."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def qk_norm_rope(x: np.ndarray, pos0=None, base: float = 10000.0, eps: float = 1e-6):
    """Forward of the prologue for one tensor x [B, T, Hx, D] (q or k): every head
    vector normalised, then rotated by its token's position."""
    B, T, _, D = x.shape
    ang = rope_angles(_positions(B, T, pos0).reshape(-1), D, base).reshape(B, T, 1, D // 2)
    return rotate(rms_norm(x, eps), ang)


def qk_norm_rope_bwd(x: np.ndarray, dy: np.ndarray, pos0=None, base: float = 10000.0,
                     eps: float = 1e-6):
    """Gradient with respect to x of sum(qk_norm_rope(x) * dy).

    The rotation is orthogonal, so the gradient at its input is the inverse rotation
    of dy.  Through the norm, with r = 1 / sqrt(mean(x^2) + eps) and x_n = r x:
    dx = r (g - x_n (x_n . g) / D) when eps = 0; in general the second term carries
    r^2 x (x . g) / D, which is written below without assuming eps = 0.
    """
    B, T, _, D = x.shape
    ang = rope_angles(_positions(B, T, pos0).reshape(-1), D, base).reshape(B, T, 1, D // 2)
    g = rotate(dy, -ang)                      # back through the rotation
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return r * g - (r ** 3) * x * np.sum(x * g, axis=-1, keepdims=True) / D
