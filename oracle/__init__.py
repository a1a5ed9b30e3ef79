"""CPU oracle for FastGen's head-wise profiling, compaction and decode.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow fp64 restatement of
what the method computes.  It shares no code with the HIP library and imports
nothing from it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does.
"""
from .fastgen_ref import (  # noqa: F401
    LEVEL_FREQUENT,
    LEVEL_FULL,
    LEVEL_LOCAL,
    LEVEL_PUNCT,
    LEVEL_SPECIAL,
    HeadProfile,
    budgets,
    causal_attention_rows,
    column_scores,
    compact_head,
    decode_incremental,
    decode_masked,
    frequent_set,
    kept_positions,
    key_levels,
    profile_head,
    profile_layer,
    recovery_from_bins,
    row_bins,
    select_policy,
)
