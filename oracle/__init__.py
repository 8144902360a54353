"""fp64 CPU oracle for paged causal grouped-query attention and the projections around it
(test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    attention,
    bf16_to_f64,
    decode,
    gather_logical,
    kv_append,
    lse_merge,
    page_of,
    prefill_chunk,
)
from .projection import o_proj, qkv_proj, round_to_bf16_bits  # noqa: F401
