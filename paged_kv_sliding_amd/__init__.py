"""Sliding-window attention over a paged KV cache for AMD Instinct MI355X.

The compute path is the C-ABI library ``libpkvs.so`` (hand-written HIP
kernels for gfx950, declared in ``include/pkvs.h``).  ``paged_kv_sliding_amd.pkvs``
is its Python binding (importing it fails when the library is not built);
``paged_kv_sliding_amd.synth`` draws seeded synthetic inputs; the library is
built by ``paged_kv_sliding_amd.build``.
"""
__all__ = ["pkvs", "synth", "build"]
