"""SparSTAR selected-block attention on AMD Instinct MI355X (gfx950).

The hot path -- block means, aggregated block scores, clip-aware joint top-k
selection and block-sparse flash-attention forward -- runs in hand-written HIP
kernels of ``libsparstar.so`` (C ABI in include/sparstar.h).  This package is
the thin Python binding over it.
"""
from .binding import (  # noqa: F401
    BLOCK, BF16, FP32, FUSED_MAX_NKB, OK, ERR_HIP, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, LIB_PATH,
    SparstarError, block_means, block_scores, block_sparse_attn_fwd, forced_blocks,
    kept_blocks, last_error, lib, select_blocks, select_blocks_from_means, select_blocks_from_means_noalloc,
    select_blocks_from_qk,
    select_workspace, select_workspace_bytes, sparse_attention, version,
    retained_mass, selection_retained_mass, transfer_scores, transferred_selection,
    token_topk_bound,
)
