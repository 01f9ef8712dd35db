"""CPU fp64 oracle for causal sliding-window attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package never imports the product.

What it computes is the plain definition of masked scaled-dot-product
attention, written out in NumPy float64 (see ``oracle/attention.py``).
"""

from .attention import (  # noqa: F401
    visible_mask,
    attn_fwd,
    attn_bwd,
    attn_decode,
    head_fwd,
    head_bwd,
    head_probs,
)
