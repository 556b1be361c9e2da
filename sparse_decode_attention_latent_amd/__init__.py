"""BasisKV decode-time sparse attention over Value latents, for MI355X (gfx950).

The compute path is the C-ABI library ``libbasiskv.so`` (hand-written HIP
kernels, declared in include/basiskv.h); ``api`` is its thin Python binding.
``configs`` and ``synth`` describe and generate the seeded synthetic
workloads; ``layout`` packs logical caches into the paged pools.  Importing
this package loads nothing: the library is opened on first use of ``api``.
"""
