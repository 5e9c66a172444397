"""fp64 CPU oracle for split-KV decode attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code with the HIP library or its binding.
"""

from .core import (  # noqa: F401
    NEG_INF,
    attention,
    attention_tokens,
    default_scale,
    gather,
    kept_tokens,
    kv_head_of,
    merge,
    merge_partials,
    micro_attention,
    micro_tokens,
    scores,
    to_f64,
)
