"""CPU oracle for unified paged attention (fp64 numpy + a 50-digit brute force).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` and by nothing else.  It shares no
code with the GPU library in ``paged_kv_cache_unified_amd``.
"""

from .attention import (  # noqa: F401
    attend_rows,
    cache_write,
    decode_e4m3fn,
    encode_e4m3fn,
    gather_context,
    merge_lse,
    paged_attention,
    paged_attention_rows,
)
