"""Block-sparse global attention for multi-view geometry transformers on MI355X.

Selection (pooled top-k, cumulative pooled mass, drift score with swap
restoration, or value-aware demand with cross-layer pair memory), the
block-sparse attention forward and the dense attention of the camera/register
query rows run in the HIP kernels of libbsgm.so; this package is the thin
ctypes binding to its C ABI (include/bsgm.h).
"""
from ._lib import (  # noqa: F401
    BEST_SWAP, BF16, CDF, DRIFT, DROPPED_SUM, F32, RENORMALISED, RERANK, RERANK_TRACK_BEST, TOPK,
    VASC, BsgmError, EXPORTS, LIB_PATH,
    attn_prepare, attn_workspace_bytes, col_capacity, drift_scores, drift_streamed_workspace_bytes,
    fused_workspace_bytes, library,
    NOALLOC_SCRATCH_BYTES, pool_blocks, pool_blocks2, select_blocks, select_blocks_fused,
    select_blocks_noalloc,
    select_blocks_pooled, select_drift_streamed, sparse_attn_fwd, special_rows_dense_fwd, special_rows_workspace_bytes,
    vasc_pairs, vasc_select_blocks, version, workspace_bytes,
)
