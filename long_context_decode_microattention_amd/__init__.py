"""Split-KV decode attention over a paged KV cache, for MI355X (gfx950).

The compute path is the HIP library ``libda.so`` built from ``csrc/``; the
binding in ``_lib`` marshals torch tensors into its C ABI (``include/da.h``)
and raises if the library is missing -- there is no other implementation.
"""

from ._lib import (  # noqa: F401
    DaError,
    DaShape,
    attention,
    attention_fp8,
    attention_workspace_size,
    check_inputs,
    load,
    merge,
    merge_partials,
    micro_attention,
    stream_read,
)
