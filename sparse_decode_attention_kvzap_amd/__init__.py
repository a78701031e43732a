"""Learned KV-cache eviction and GQA decode attention over the pruned, paged cache,
for AMD Instinct MI355X (gfx950).

The compute path is libkvp.so (hand-written HIP kernels behind the C ABI in
include/kvp.h); this package is its thin ctypes binding plus the in-tree build.
"""
from ._lib import (  # noqa: F401
    KVP_BF16, KVP_COMPACT_DEMOTE_INT8, KVP_COMPACT_EVICT, KVP_F32, KVP_PAGE,
    KVP_SCORER_LINEAR, KVP_SCORER_MLP, ERR_POOL8_FULL, ERR_POOL_FULL, ERR_TABLE_FULL,
    KVP_LP_INT8, KVP_LP_INT4, KVP_LP_FP8_E4M3,
    KvpError, PagedKV, Ring, Scorer, decode_attn_workspace, kvp_check, kvp_clear_error,
    kvp_compact, kvp_compact_workspace_size, kvp_decode_attn,
    kvp_decode_attn_workspace_size, kvp_decode_attn_noalloc, KVP_NOALLOC_SCRATCH_BYTES,
    kvp_decode_step, kvp_decode_step_workspace_size, decode_step_workspace,
    kvp_prefill_attn, kvp_reset, kvp_score,
    kvp_score_workspace_size,
    kvp_select, kvp_select_workspace_size, kvp_status_str, kvp_step_delayed,
    kvp_score_step_delayed,
    kvp_threshold, kvp_threshold_workspace_size, kvp_version,
    load, sm_scale, LIB_PATH,
)
