"""fp64 CPU oracle for paged causal grouped-query attention (test infrastructure only).

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
