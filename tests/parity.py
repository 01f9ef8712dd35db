"""Helpers for comparing the HIP path with the fp64 oracle (imported by GPU tests)."""

import numpy as np
import torch

# Tolerances (max-abs on each output tensor; bf16 also bounds the relative L2 error).
TOL_F32 = 1e-5
TOL_BF16_ABS = 2e-2
TOL_BF16_REL = 5e-3
TOL_BF16_LSE = 1e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mask = ~np.isnan(ref)
    d = got[mask] - ref[mask]
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref[mask]))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else 0.0
    return max_abs, rel, float(np.abs(ref[mask]).max()) if d.size else 0.0


def check(name, got, ref, dtype, lse=False, out_ulp=False):
    """Assert the tolerance for one output; returns (max_abs, rel_l2).

    ``out_ulp`` (bf16 sums over several heads, whose magnitude can pass 8): the
    max-abs bar applies elementwise on top of the output's own bf16 rounding,
    |got - ref| <= 2e-2 + 2^-9 |ref| (half an ulp of a bf16 value is at most
    2^-9 of it); the relative-L2 bar is unchanged."""
    got = f64(got) if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(got[~np.isnan(ref)])), f"{name}: non-finite output"
    max_abs, rel, ref_max = errors(got, ref)
    if out_ulp and dtype == torch.bfloat16:
        mask = ~np.isnan(ref)
        excess = float((np.abs(got[mask] - ref[mask]) - 2.0 ** -9 * np.abs(ref[mask])).max())
        assert excess <= TOL_BF16_ABS, (
            f"{name}: max(|err| - 2^-9 |ref|) {excess:.3e} > {TOL_BF16_ABS} (|ref| <= {ref_max:.2f})")
        assert rel <= TOL_BF16_REL, f"{name}: rel-L2 {rel:.3e} > {TOL_BF16_REL}"
        return max_abs, rel
    if dtype == torch.float32:
        assert max_abs <= TOL_F32, f"{name}: max-abs {max_abs:.3e} > {TOL_F32} (|ref| <= {ref_max:.2f})"
    elif lse:
        assert max_abs <= TOL_BF16_LSE, f"{name}: max-abs {max_abs:.3e} > {TOL_BF16_LSE}"
    else:
        assert max_abs <= TOL_BF16_ABS, f"{name}: max-abs {max_abs:.3e} > {TOL_BF16_ABS} (|ref| <= {ref_max:.2f})"
        assert rel <= TOL_BF16_REL, f"{name}: rel-L2 {rel:.3e} > {TOL_BF16_REL}"
    return max_abs, rel


def sample_heads(B, H, n, seed=0):
    """First, last and random (b, h) pairs."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (B - 1, H - 1)}
    while len(pairs) < min(n, B * H):
        pairs.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(pairs)


def only_heads(a, heads, layout="bthd"):
    """Copy of `a` with every head not in `heads` set to NaN (for sampled comparisons)."""
    out = np.full_like(np.asarray(a, np.float64), np.nan)
    for b, h in heads:
        if layout == "bthd":
            out[b, :, h, :] = a[b, :, h, :]
        else:  # bht
            out[b, h, :] = a[b, h, :]
    return out
