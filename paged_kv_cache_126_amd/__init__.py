"""Paged decode attention and KV append for AMD MI355X (gfx950).

``lib`` binds the HIP library's C ABI; ``block_manager`` is the host-side
frame pool and block tables that feed it.
"""
from .block_manager import AppendResult, BlockPool, SeqManager
from .block_manager import PrefixCachingSeqManager
from .lib import (PA_MAX_GROUP, PA_PREFILL_TILE, PagedAttnError, alloc_workspace, kernel_timing,
                  kv_append,
                  kv_copy_blocks, load, paged_attn_decode, paged_attn_decode_grouped,
                  paged_attn_decode_noalloc,
                  paged_attn_prefill, paged_gather, partition_tokens, workspace_size)

__all__ = [
    "PA_MAX_GROUP", "PA_PREFILL_TILE", "AppendResult", "BlockPool", "SeqManager", "PrefixCachingSeqManager", "PagedAttnError",
    "alloc_workspace", "kernel_timing", "kv_append", "kv_copy_blocks",
    "load", "paged_attn_decode", "paged_attn_decode_grouped", "paged_attn_decode_noalloc", "paged_attn_prefill", "paged_gather",
    "partition_tokens", "workspace_size",
]
