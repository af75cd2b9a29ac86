"""Plain fp64 CPU oracle for the SparSTAR hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here.
"""
from .sparstar_oracle import (  # noqa: F401
    decode, block_means, block_scores, forced_blocks, budget, kept_blocks,
    select_blocks, select_row, sparse_attention, sparse_attention_rows,
    run_pipeline, selected_flops, retained_mass_rows, token_topk_bound_rows,
    transfer_query_map, transfer_key_map, transfer_scores, transferred_selection,
)
