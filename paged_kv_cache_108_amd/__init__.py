"""pkv: paged decode attention and the KV-cache write for AMD MI355X (gfx950).

The computation lives in ``libpkv.so`` (hand-written HIP kernels and a C++
host allocator, C ABI in ``include/pkv.h``); this package only passes
arguments to it. ``workloads`` draws the seeded synthetic inputs.
"""

from .api import (kv_cache_write, copy_blocks, paged_decode_attn, paged_decode_step, paged_decode_step_noalloc,
                  paged_decode_plan_workers, build_paged_decode_plan, paged_decode_step_planned, DecodePlan,
                  build_paged_window_plan, paged_multi_query_attn_planned, WindowPlan, plan_mark_shared_blocks,
                  stream_read, paged_gather_read, paged_decode_attn_workspace_size,
                  paged_decode_attn_workspace, paged_multi_query_attn,
                  paged_multi_query_attn_workspace, Allocator,
                  slots_from_tables, waste_stats, block_hashes, last_error, version, quantise_pool, PkvError,
                  NoBlocks, PKV_PARTITION_BALANCED, paged_decode_attn_lse, paged_shared_prefix_attn,
                  merge_attn_states, shared_prefix_plan, SharedPrefixDecode, v_shape_ok,
                  paged_shared_prefix_decode, paged_shared_prefix_decode_workspace)
from ._lib import lib, LIB_PATH, SIGNATURES, PKV_F32, PKV_BF16, PKV_FP8_E4M3

__all__ = [
    "kv_cache_write", "copy_blocks", "paged_decode_attn", "paged_decode_step", "paged_decode_step_noalloc",
    "paged_decode_plan_workers", "build_paged_decode_plan", "paged_decode_step_planned", "DecodePlan",
    "build_paged_window_plan", "paged_multi_query_attn_planned", "WindowPlan", "plan_mark_shared_blocks",
    "stream_read", "paged_gather_read", "paged_decode_attn_workspace_size",
    "paged_decode_attn_workspace", "paged_multi_query_attn", "paged_multi_query_attn_workspace",
    "Allocator",
    "slots_from_tables", "waste_stats", "block_hashes", "last_error", "version", "quantise_pool", "PkvError",
    "NoBlocks", "PKV_PARTITION_BALANCED", "paged_decode_attn_lse", "paged_shared_prefix_attn",
    "merge_attn_states", "shared_prefix_plan", "SharedPrefixDecode",
    "paged_shared_prefix_decode", "paged_shared_prefix_decode_workspace", "v_shape_ok", "lib", "LIB_PATH", "SIGNATURES", "PKV_F32", "PKV_BF16", "PKV_FP8_E4M3",
]
