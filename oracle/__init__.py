"""fp64 CPU oracle for Forecast-driven block-sparse attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the HIP library, and it imports nothing
from the library.
"""
from .sparda_ref import (  # noqa: F401
    Selection,
    attend_decode,
    attend_prefill,
    block_cache_plan,
    block_sets,
    decode_select,
    decode_select_windows,
    decode_step_lookahead,
    forecast_proj,
    gather_selected_blocks,
    kth_gap,
    kv_block_meanpool,
    kv_window_meanpool,
    multihead_select_decode,
    prefill_select,
    prefill_select_pooled,
    prefill_select_windows,
    qkvf_proj,
    qkvf_proj_prefill,
    rank_topk,
    window_block_scores,
)
