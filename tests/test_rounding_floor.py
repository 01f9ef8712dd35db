"""How much of the bf16 bar the rounding of the forward's output alone uses up.

A composed training step feeds the backward the forward's o rounded to bf16, and
delta = dO . o is formed from that rounded o.  Here the oracle's gradient with delta
from the bf16-rounded exact o is compared with the exact gradient, on the edge sweep
that the composed GPU test runs (tests/parity.py).  The cases where it already misses
the bar are exactly ``COMPOSED_ROUNDING_MISSES``: there no kernel, however exact, can
meet the bar against the exact gradient, and the composed GPU test skips them.  Every
other case leaves room for the kernels' own rounding.
"""

import itertools
import math

import numpy as np
import torch

from causal_sliding_window_amd import inputs
from oracle import attention as orc
from parity import (COMPOSED_ROUNDING_MISSES, EDGE_D, EDGE_T, EDGE_W, TOL_BF16_ABS,
                    TOL_BF16_REL, edge_inputs, errors)


def _rounded_o_gradient_errors(T, W, D):
    x = edge_inputs(inputs, T, W, D)
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    scale = 1 / math.sqrt(D)
    ro, _ = orc.attn_fwd(a["q"], a["k"], a["v"], W, scale)
    exact = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], W, scale)
    o16 = inputs.to_f64(torch.from_numpy(ro).to(torch.bfloat16))
    rounded = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], W, scale, o=o16)
    return {n: errors(g, r)[:2] for n, g, r in zip(("dq", "dk", "dv"), rounded, exact)}


def test_rounded_output_misses_are_the_skipped_cases():
    misses, worst = set(), {}
    for T, W, D in itertools.product(EDGE_T, EDGE_W, EDGE_D):
        for n, (max_abs, rel) in _rounded_o_gradient_errors(T, W, D).items():
            if max_abs > TOL_BF16_ABS or rel > TOL_BF16_REL:
                misses.add((T, W, D))
                worst[(T, W, D, n)] = (max_abs, rel)
    assert misses == COMPOSED_ROUNDING_MISSES, worst


def test_exact_output_leaves_the_gradient_exact():
    """Control: with delta from the exact (unrounded) o the same comparison is exact to
    fp64 rounding, so the misses above come from rounding o alone."""
    x = edge_inputs(inputs, 2, 63, 64)
    a = {n: inputs.to_f64(t) for n, t in x.items()}
    scale = 1 / math.sqrt(64)
    ro, _ = orc.attn_fwd(a["q"], a["k"], a["v"], 63, scale)
    exact = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], 63, scale)
    same = orc.attn_bwd(a["q"], a["k"], a["v"], a["do"], 63, scale, o=ro)
    for g, r in zip(same, exact):
        assert np.abs(g - r).max() <= 1e-12
