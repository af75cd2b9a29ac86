"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
the acceptance rules, and row sampling.  The rules are the ones the tests
enforce:
  * selection: bit-exact, except that a block kept by only one side is
    tolerated when the oracle's scores of the swapped blocks differ by no more
    than 1e-6 relative to max(|S_j|, |S_j'|, 1e-3 * max_row |S|);
  * fp32 outputs: max |diff| <= 1e-4;
  * bf16 outputs: max |diff| <= 2e-2 and ||diff||_2 / ||ref||_2 <= 1e-2.
"""
import math
import sys

import numpy as np
import torch

import oracle

TOL_FP32_MAXABS = 1e-4
TOL_BF16_MAXABS = 2e-2
TOL_BF16_RELL2 = 1e-2
TIE_REL = 1e-6


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_selection(S, n_forced, density, g_count, g_index):
    """S: oracle fp64 scores [..., nqb, nkb]; g_*: GPU results (numpy).
    Returns the number of rows with a tolerated near-tie swap."""
    nkb = S.shape[-1]
    rows = S.reshape(-1, nkb)
    gc = np.asarray(g_count).reshape(-1)
    gi = np.asarray(g_index).reshape(gc.size, -1)
    k = oracle.budget(nkb - n_forced, density)
    swaps = 0
    for r in range(rows.shape[0]):
        sel = oracle.select_row(rows[r], n_forced, density)
        assert gc[r] == sel.size, (r, gc[r], sel.size)
        got = gi[r, :gc[r]]
        assert np.all(gi[r, gc[r]:] == -1), r
        assert np.all(np.diff(got) > 0), r
        assert np.array_equal(got[:n_forced], np.arange(n_forced)), r
        if np.array_equal(got, sel):
            continue
        only_o = np.setdiff1d(sel, got)
        only_g = np.setdiff1d(got, sel)
        assert only_o.size == only_g.size and only_o.size > 0, r
        assert np.all(only_g >= n_forced) and np.all(only_g < nkb), r
        s = rows[r]
        hi = s[only_o].max()          # oracle kept, GPU dropped
        lo = s[only_g].min()          # GPU kept, oracle dropped
        elig = s[n_forced:]
        scale = max(abs(hi), abs(lo), 1e-3 * np.nanmax(np.abs(elig)))
        assert hi - lo <= TIE_REL * scale, (r, hi, lo, k)
        swaps += 1
    return swaps


def compare_outputs(o_gpu, o_ref, dtype, what=""):
    diff = np.abs(o_gpu - o_ref)
    mx = float(diff.max()) if diff.size else 0.0
    if dtype == "fp32":
        assert mx <= TOL_FP32_MAXABS, (what, mx)
        return mx, None
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    assert mx <= TOL_BF16_MAXABS and rel <= TOL_BF16_RELL2, (what, mx, rel)
    return mx, rel


def compare_lse(l_gpu, l_ref, tol, what=""):
    both_inf = np.isneginf(l_gpu) & np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), np.isneginf(l_ref)), what
    d = np.abs(np.where(both_inf, 0.0, l_gpu) - np.where(both_inf, 0.0, l_ref))
    assert float(d.max(initial=0.0)) <= tol, (what, float(d.max()))


def sample_rows(B, H, nqb, kv_count, kv_index, nkb, n=24, seed=0):
    """Deterministic sample of (b, h, i) rows: first and last query blocks, rows
    that keep the (possibly partial) last key block, and random rows."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, H - 1, nqb - 1), (0, H // 2, nqb - 1)}
    cnt = kv_count.reshape(B, H, nqb)
    idx = kv_index.reshape(B, H, nqb, -1)
    hits = np.argwhere((idx == nkb - 1).any(axis=-1))
    for t in hits[:3]:
        rows.add(tuple(int(x) for x in t))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nqb))))
    return sorted(rows)
