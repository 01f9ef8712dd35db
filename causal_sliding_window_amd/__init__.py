"""libswattn: causal sliding-window attention for AMD Instinct MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI (``include/swattn.h``,
built as ``causal_sliding_window_amd/libswattn.so``).  ``causal_sliding_window_amd.swattn``
is the thin Python binding (argument marshalling only); ``inputs`` draws the seeded
synthetic workloads.  Importing this package loads nothing; the binding loads the
library on first use and raises if it is missing.
"""
