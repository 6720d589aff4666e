"""MI355X-native Gated DeltaNet + HLA hot path.

The compute lives in ``libhla.so`` (hand-written HIP kernels for gfx950 behind a C ABI,
declared in ``include/hla.h``).  ``gated_deltanet_hybrid_amd.hla`` is the thin Python
binding; importing this package does not load the library, so host-only modules
(``inputs``, ``layout``) work on machines without a GPU.
"""
__all__ = ["inputs", "layout"]
