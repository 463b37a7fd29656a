"""Paged decode attention and KV append for AMD MI355X (gfx950).

``lib`` binds the HIP library's C ABI; ``native_blocks`` binds the host-side
frame pool and block tables (C++) that feed it; ``driver`` plays schedules
through both.
"""
from .lib import (PA_MAX_GROUP, PA_PREFILL_TILE, PagedAttnError, alloc_workspace, kernel_timing,
                  kv_append, kv_copy_blocks, load, paged_attn_decode, paged_attn_decode_grouped,
                  paged_attn_decode_noalloc, paged_attn_prefill, paged_gather, partition_tokens,
                  workspace_size)
from .native_blocks import AppendResult, NativeBlockManager

__all__ = [
    "PA_MAX_GROUP", "PA_PREFILL_TILE", "AppendResult", "NativeBlockManager", "PagedAttnError",
    "alloc_workspace", "kernel_timing", "kv_append", "kv_copy_blocks", "load", "paged_attn_decode",
    "paged_attn_decode_grouped", "paged_attn_decode_noalloc", "paged_attn_prefill", "paged_gather",
    "partition_tokens", "workspace_size",
]
