"""Split-KV decode attention over a paged KV cache, for MI355X (gfx950).

The compute path is the HIP library ``libda.so`` built from ``csrc/``; the
binding in ``_lib`` marshals torch tensors into its C ABI (``include/da.h``).
"""
