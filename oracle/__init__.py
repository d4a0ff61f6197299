"""fp64 CPU oracle of MoBA causal prefill (forward and backward) and decode (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg use
this package. It shares no code with the HIP library and imports nothing from it.
"""
from .moba_oracle import (  # noqa: F401
    attended_count,
    attended_keys,
    attended_pairs_closed_form,
    gate_scores,
    moba_backward_ref,
    moba_backward_ref_varlen,
    moba_decode_ref,
    moba_ref,
    moba_ref_varlen,
    n_blocks,
    pooled_keys,
    pooled_keys_fp32,
    query_lists,
    select_blocks,
    select_row,
    sparsity,
    topk_for_sparsity,
    POOLINGS,
)
