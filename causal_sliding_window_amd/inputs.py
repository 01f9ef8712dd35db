"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only draws tensors.  Both the HIP
path and the fp64 oracle are fed from it (the oracle receives the exact rounded
values, upcast to float64).

Recipe (the pages give no data for the kernel itself; every tensor is synthetic):

* q, k, v, dO ~ N(0, 1), drawn in float32 on the CPU with ``torch.Generator``
  seeded ``s, s+1, s+2, s+3`` for q, k, v, dO respectively.
* With ``qk_norm`` (the nanochat model's parameter-free QK RMS norm, listed among
  the architecture features of the nanochat launch article and of section 1 of
  the nanochat guide), every q and k head vector is divided by its RMS over D
  (eps = 0) in float32.  v and dO stay N(0, 1).
* The float32 values are then rounded to the target dtype (bf16 round-to-nearest-
  even, or kept as float32).
* Decode: cache lengths ``numpy.random.default_rng(7).integers(512, 4096,
  endpoint=True, size=B)``; q [B, H, D] and the full K/V caches
  [B, Tmax, H, D] ~ N(0, 1) from torch seeds 7, 8, 9 (rows past a sequence's
  length are drawn too and never read).
"""

from __future__ import annotations

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}

# Named workloads.  Each training config lists the windows of the layers it runs
# (-1 = full causal); "mid-alt" runs four layers that alternate a short and a
# long window, the per-layer pattern of the nanochat guide's section 1.
CONFIGS = {
    "tiny": dict(kind="train", B=1, H=2, T=128, D=64, dtype="f32",
                 windows=[-1], seeds=[0], qk_norm=False),
    "small": dict(kind="train", B=8, H=6, T=2048, D=128, dtype="bf16",
                  windows=[-1], seeds=[0], qk_norm=True),
    "mid-alt": dict(kind="train", B=4, H=12, T=2048, D=128, dtype="bf16",
                    windows=[512, 2048, 512, 2048], seeds=[0, 4, 8, 12],
                    qk_norm=True),
    "wide-sw": dict(kind="train", B=2, H=16, T=4096, D=128, dtype="bf16",
                    windows=[256], seeds=[0], qk_norm=True),
    # the guide's "SSSL" layer pattern (three short-window layers, then one long) at the
    # mid model's shape; the pages give no window sizes: short = T / 4 (as mid-alt's
    # short layers), long = full causal
    "sssl": dict(kind="train", B=4, H=12, T=2048, D=128, dtype="bf16",
                 windows=[512, 512, 512, 2048], seeds=[0, 4, 8, 12], qk_norm=True),
    "decode": dict(kind="decode", B=32, H=12, D=128, Tmax=4096, dtype="bf16",
                   windows=[-1, 1024], len_seed=7, len_lo=512, len_hi=4096,
                   seed=7),
}


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _rms_normalize(x: torch.Tensor) -> torch.Tensor:
    return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True))


def training_inputs(B: int, T: int, H: int, D: int, dtype: str = "bf16",
                    seed: int = 0, qk_norm: bool = False, Hkv: int | None = None) -> dict:
    """q, dO as CPU tensors [B, T, H, D] and k, v [B, T, Hkv, D] (Hkv = H by default) in
    ``dtype`` ("bf16" or "f32")."""
    shape = (B, T, H, D)
    kv_shape = (B, T, H if Hkv is None else Hkv, D)
    q = _randn(shape, seed)
    k = _randn(kv_shape, seed + 1)
    v = _randn(kv_shape, seed + 2)
    do = _randn(shape, seed + 3)
    if qk_norm:
        q = _rms_normalize(q)
        k = _rms_normalize(k)
    td = DTYPES[dtype]
    return {"q": q.to(td), "k": k.to(td), "v": v.to(td), "do": do.to(td)}


def decode_lengths(B: int, seed: int = 7, lo: int = 512, hi: int = 4096) -> np.ndarray:
    """Per-sequence cache lengths, uniform integers in [lo, hi] (int32)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, endpoint=True, size=B).astype(np.int32)


def decode_inputs(B: int, H: int, D: int, Tmax: int, dtype: str = "bf16",
                  seed: int = 7, lengths=None, Hkv: int | None = None) -> dict:
    """q [B, H, D], k/v caches [B, Tmax, Hkv, D] (Hkv = H by default) and int32
    seqlens [B] (CPU)."""
    td = DTYPES[dtype]
    if lengths is None:
        lengths = decode_lengths(B, seed=7, lo=min(512, Tmax), hi=Tmax)
    seqlens = torch.as_tensor(np.asarray(lengths, dtype=np.int32))
    q = _randn((B, H, D), seed).to(td)
    Hkv = H if Hkv is None else Hkv
    k = _randn((B, Tmax, Hkv, D), seed + 1).to(td)
    v = _randn((B, Tmax, Hkv, D), seed + 2).to(td)
    return {"q": q, "k_cache": k, "v_cache": v, "seqlens": seqlens}


def config_inputs(name: str, layer: int = 0) -> dict:
    """Inputs of a named workload (one layer of a training config)."""
    c = CONFIGS[name]
    if c["kind"] == "decode":
        lengths = decode_lengths(c["B"], c["len_seed"], c["len_lo"], c["len_hi"])
        return decode_inputs(c["B"], c["H"], c["D"], c["Tmax"], c["dtype"],
                             c["seed"], lengths)
    return training_inputs(c["B"], c["T"], c["H"], c["D"], c["dtype"],
                           c["seeds"][layer], c["qk_norm"])


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (CPU or device) tensor to a float64 NumPy array."""
    return x.detach().to("cpu", torch.float64).numpy()
