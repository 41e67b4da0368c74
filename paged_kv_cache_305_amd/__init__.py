"""MI355X (gfx950) paged decode attention.

The data-parallel hot path of PagedAttention as a C-ABI library
(``libpagedattn.so``, declared in ``include/pagedattn.h``) with this thin
Python binding:

  * ``paged_attention_decode`` -- single-query attention read through
    per-sequence block tables (HIP kernels; MFMA for grouped-query heads);
  * ``paged_attention_decode_prefix`` -- the same with a prefix shared by
    every sequence read once for all of them;
  * ``paged_attention_decode_noalloc`` -- the decode step with the
    library's own device scratch instead of a workspace (allocates nothing);
  * ``reshape_and_cache`` -- write new tokens' K/V into their slots;
  * ``copy_blocks`` -- the copy of copy-on-write;
  * ``reshape_and_cache_layers``, ``copy_blocks_layers`` -- both over every
    layer's pools in one launch;
  * ``swap_blocks`` -- block copies between GPU and pinned host pools;
  * ``BlockAllocator`` -- host free list, refcounts, copy-on-write and a
    swap space for preempted sequences.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, PA_BF16, PA_ERR_HIP, PA_ERR_INVALID_ARG, PA_ERR_OUT_OF_BLOCKS,
    PA_DECODE_KV_REUSED, PA_ERR_UNKNOWN_SEQ, PA_ERR_UNSUPPORTED, PA_FP32, PA_OK,
    PA_PARTITION_AUTO, PA_PARTITION_BALANCED, PA_AUTO_WHOLE_MAX_LEN, BlockAllocator,
    PagedAttnError, resolve_partition,
    allocate_pools, copy_blocks, key_cache_shape, load, paged_attention_decode,
    paged_attention_workspace_bytes, reshape_and_cache, set_balance_weights, set_timing_events,
    swap_blocks, value_cache_shape, pointer_array, reshape_and_cache_layers, copy_blocks_layers,
    paged_attention_decode_prefix, paged_attention_prefix_workspace_bytes,
    paged_attention_decode_noalloc)
