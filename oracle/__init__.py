"""FP64 CPU oracle for causal prefill attention -- test infrastructure only.

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the library or its binding.
"""
from .attention import (  # noqa: F401
    attention_chunked,
    attention_decode,
    attention_head,
    attention_paged,
    attention_rows,
    attention_varlen,
    gather_pages,
    kv_head_of,
    softmax_probs,
    visibility,
    visible_pairs,
)
