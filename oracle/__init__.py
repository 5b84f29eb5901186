"""CPU oracle (float64) for the fused attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and imports nothing from it; see ``oracle/ref.py`` for what it computes and
the passages it follows.
"""
from .ref import (  # noqa: F401
    softmax_attend, causal_visible, window_visible, rope_rotate, kv_head_of, gather_pages,
    ref_decode_paged, ref_decode_paged_fp8, fp8_e4m3_to_float, ref_prefill_varlen,
    ref_prefill_paged,
    merge_states, error_stats,
)
