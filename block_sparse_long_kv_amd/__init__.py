"""Python binding of libbskv (Forecast-driven block-sparse attention, gfx950).

Argument marshalling only: every step runs in the HIP kernels of
libbskv.so.  torch supplies device memory and the current stream.  The
functions carry the names of the C ABI in include/bskv.h without the
``bskv_`` prefix; see that header for layouts and semantics.

Importing this package fails loudly when libbskv.so has not been built
(``python block_sparse_long_kv_amd/build.py``).
"""
from ._lib import (  # noqa: F401
    BlockCache,
    BskvError,
    block_cache_plan,
    block_sparse_attn_decode,
    block_sparse_attn_decode_cached,
    block_sparse_attn_decode_cached_fill,
    block_sparse_attn_prefill,
    decode_layer_lookahead,
    decode_layer_lookahead_noalloc,
    forecast_block_score_topk,
    forecast_block_score_topk_pooled,
    forecast_proj,
    forecast_window_score_topk,
    host_device_pointer,
    kv_block_meanpool,
    kv_window_meanpool,
    lib,
    multihead_block_score_topk,
    prefetch_cache_fill,
    prefetch_selected_blocks,
    qkvf_proj_decode,
    qkvf_proj_prefill,
    workspace_bytes,
)
