"""The allocation-free score + selection entry point
(sparstar_select_blocks_from_means_noalloc, through the C ABI) selects exactly
what the workspace entry point (sparstar_select_blocks_from_means) selects, on
two calls in a row, the second on a smaller input, with the library's own
device scratch standing in for the workspace."""
import numpy as np
import pytest
import torch

import block_sparse_attention_head_amd as sp
from tests.parity_util import log

pytestmark = pytest.mark.gpu

CALLS = [
    # B, H, nqb, nkb, D, n_forced_blocks, density: a full 72k scale's means, then a small one
    (1, 16, 563, 1129, 128, 4, 0.09375),
    (2, 3, 37, 131, 64, 2, 0.25),
]


def _means(B, H, nqb, nkb, D, seed):
    rng = np.random.default_rng(seed)
    qb = (rng.standard_normal((B, H, nqb, D)) * 0.3).astype(np.float32)
    kb = (rng.standard_normal((B, H, nkb, D)) * 0.3).astype(np.float32)
    return torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    for n, (B, H, nqb, nkb, D, F, density) in enumerate(CALLS):
        log(f"noalloc call {n}: B={B} H={H} nqb={nqb} nkb={nkb} D={D} F={F} density={density}, "
            f"workspace {sp.select_workspace_bytes(B, H, nqb, nkb)} bytes")
        q, k = _means(B, H, nqb, nkb, D, seed=100 + n)
        ref_cnt, ref_idx = sp.select_blocks_from_means(q, k, F, density)
        cnt = torch.full_like(ref_cnt, -7)
        idx = torch.full_like(ref_idx, -7)
        sp.select_blocks_from_means_noalloc(q, k, F, density, kv_count=cnt, kv_index=idx)
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref_cnt), n
        assert torch.equal(idx, ref_idx), n
        log(f"  identical on {cnt.numel()} rows")
