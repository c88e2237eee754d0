"""CSA2 compressed sparse attention on MI355X (gfx950).

The product is the C-ABI library ``libcsa2.so`` (declared in include/csa2.h)
and its thin ctypes binding ``sparse_long_context_amd.csa2``.  ``synth`` draws
the seeded synthetic workloads.
"""
