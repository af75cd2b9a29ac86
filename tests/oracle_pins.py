"""Checks that pin the oracle to facts outside itself.

Each check takes an implementation namespace ``impl`` exposing the oracle's
functions, so the same checks can be run against deliberately broken copies
(tests/test_oracle_mutations.py) to show that they catch plausible mistakes.
Every check raises AssertionError on failure.
"""
import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- identity: block-mean dot product == average pairwise logit ------------
def pin_identity(impl, seed=0):
    """The review ('What carries the argument') notes that the inner product of
    two block means is the mean, over all token pairs of the two blocks, of
    the unscaled logit q_t . k_s.  Checked by brute force over token pairs."""
    rng = np.random.default_rng(seed)
    for D in (4, 64):
        for ni, nj in [(1, 1), (3, 1), (1, 3), (3, 64), (64, 128), (128, 128), (128, 3)]:
            block = 128
            q = rng.standard_normal((ni, D)) + rng.standard_normal(D)
            k = rng.standard_normal((nj, D)) - rng.standard_normal(D)
            S = impl.block_scores(impl.block_means(q, block), impl.block_means(k, block))
            assert S.shape == (1, 1)
            if ni * nj <= 64:   # small: pure-Python double loop over token pairs
                tot = math.fsum(math.fsum(q[t, d] * k[s, d] for d in range(D))
                                for t in range(ni) for s in range(nj))
                avg = tot / (ni * nj)
            else:
                avg = float((q @ k.T).mean())
            lhs = S[0, 0] * math.sqrt(D)
            assert abs(lhs - avg) <= 1e-12 * max(1.0, abs(avg)), (D, ni, nj, lhs, avg)


def pin_means_closed_form(impl):
    """Hand-worked means and scores (block = 2, D = 2, partial last block).

    Q tokens (1,2) (3,4) | (5,7)   -> qbar = (2,3), (5,7)
    K tokens (0,1) (2,-1) | (4,4)  -> kbar = (1,0), (4,4)
    S = D^-1/2 * qbar kbar^T = [[2, 20], [5, 48]] / sqrt(2)
    """
    q = np.array([[1., 2.], [3., 4.], [5., 7.]])
    k = np.array([[0., 1.], [2., -1.], [4., 4.]])
    qb = impl.block_means(q, 2)
    kb = impl.block_means(k, 2)
    assert np.array_equal(qb, [[2., 3.], [5., 7.]]), qb
    assert np.array_equal(kb, [[1., 0.], [4., 4.]]), kb
    S = impl.block_scores(qb, kb)
    want = np.array([[2., 20.], [5., 48.]]) / math.sqrt(2.0)
    assert np.allclose(S, want, rtol=1e-15, atol=0), S
    # batched leading dims
    x = np.arange(2 * 3 * 5 * 2, dtype=np.float64).reshape(2, 3, 5, 2)
    m = impl.block_means(x, 2)
    assert m.shape == (2, 3, 3, 2)
    assert np.array_equal(m[1, 2, 2], x[1, 2, 4])             # 1-token block
    assert np.array_equal(m[0, 1, 0], (x[0, 1, 0] + x[0, 1, 1]) / 2)


# --- selection ---------------------------------------------------------------
def _rank_select(s, n_forced, k):
    """Eligible j is kept iff fewer than k eligible blocks beat it, where j'
    beats j if S_j' > S_j, or S_j' == S_j and j' < j; NaN is beaten by every
    number and among NaNs the lower index wins."""
    nkb = len(s)
    kept = list(range(n_forced))

    def beats(a, b):
        sa, sb = s[a], s[b]
        na, nb = math.isnan(sa), math.isnan(sb)
        if na and nb:
            return a < b
        if na:
            return False
        if nb:
            return True
        return sa > sb or (sa == sb and a < b)

    for j in range(n_forced, nkb):
        better = sum(1 for jj in range(n_forced, nkb) if jj != j and beats(jj, j))
        if better < k:
            kept.append(j)
    return kept


def pin_selection_bruteforce(impl, seed=1):
    rng = np.random.default_rng(seed)
    for trial in range(300):
        nkb = int(rng.integers(1, 40))
        F_ = int(rng.integers(0, nkb + 1))
        dens = float(rng.choice([0.0, 0.09375, 0.1875, 0.25, 0.625, 1.0, 0.5]))
        s = rng.standard_normal(nkb)
        if trial % 3 == 1:      # coarse values -> many exact ties
            s = np.round(s * 2) / 2
        if trial % 5 == 2:
            s[rng.integers(0, nkb, size=max(1, nkb // 4))] = np.nan
        if trial % 7 == 3:
            s[rng.integers(0, nkb, size=max(1, nkb // 5))] = rng.choice([np.inf, -np.inf])
        k = math.ceil(dens * (nkb - F_))
        got = list(impl.select_row(s, F_, dens))
        want = _rank_select(s, F_, k)
        assert got == want, (trial, s, F_, dens, got, want)


def pin_ties_duplicated_blocks(impl):
    """Exactly duplicated key blocks give exactly equal scores; the lower index wins."""
    rng = np.random.default_rng(3)
    D, b = 8, 4
    kblocks = rng.standard_normal((6, b, D))
    kblocks[4] = kblocks[1]          # duplicate of block 1
    kblocks[5] = kblocks[2]          # duplicate of block 2
    k = kblocks.reshape(-1, D)
    q = rng.standard_normal((b, D))
    qb = impl.block_means(q, b)
    kb = impl.block_means(k, b)
    S = impl.block_scores(qb, kb)[0]
    assert S[4] == S[1] and S[5] == S[2]
    # rank with budget such that the threshold falls between duplicates
    order = sorted(range(1, 6), key=lambda j: (-S[j], j))
    for kk in range(1, 6):
        dens = kk / 5.0
        got = [j for j in impl.select_row(S, 1, dens) if j >= 1]
        assert got == sorted(order[:kk]), (kk, got, order)
        for a, c in ((1, 4), (2, 5)):
            if c in got:
                assert a in got


def pin_counts(impl, S, n_forced, density):
    nkb = S.shape[-1]
    count, index = impl.select_blocks(S, n_forced, density)
    k = math.ceil(density * (nkb - n_forced))
    assert np.all(count == n_forced + k)
    flat = index.reshape(-1, index.shape[-1])
    for r in range(flat.shape[0]):
        row = flat[r, :count.reshape(-1)[r]]
        assert np.all(row[:n_forced] == np.arange(n_forced))     # forced kept
        assert np.all(np.diff(row) > 0)                          # ascending, unique
        assert row.size == 0 or (row[0] >= 0 and row[-1] < nkb)
    if density == 1.0:
        assert np.all(count == nkb)


def pin_tiny_budget(impl):
    g = _golden("tiny_budget.json")
    assert impl.budget(g["nkb"] - g["n_forced_blocks"], g["density"]) == g["k"]
    assert impl.kept_blocks(g["nkb"], g["n_forced_blocks"], g["density"]) == g["kept"]
    assert impl.forced_blocks(128, 128) == 1
    assert impl.forced_blocks(512 + 3600, 128) == 33
    assert impl.forced_blocks(0, 128) == 0


# --- attention ---------------------------------------------------------------
def _textbook_attention(q, k, v, scale):
    """Double loop, one query at a time (small inputs only)."""
    n, D = q.shape
    out = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for t in range(n):
        logits = [scale * math.fsum(q[t, d] * k[s, d] for d in range(D)) for s in range(k.shape[0])]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = math.fsum(w)
        for d in range(v.shape[1]):
            out[t, d] = math.fsum(w[s] * v[s, d] for s in range(k.shape[0])) / z
        lse[t] = mx + math.log(z)
    return out, lse


def pin_dense_equivalence(impl, seed=4):
    """At density 1.0 every block is kept and the result is dense softmax attention."""
    rng = np.random.default_rng(seed)
    # textbook double loop, tiny
    B, H, Nq, Nk, D, b = 1, 2, 7, 11, 4, 4
    q = rng.standard_normal((B, H, Nq, D))
    k = rng.standard_normal((B, H, Nk, D))
    v = rng.standard_normal((B, H, Nk, D))
    res = impl.run_pipeline(q, k, v, n_forced_tokens=3, density=1.0, block=b)
    scale = 1 / math.sqrt(D)
    for h in range(H):
        o_ref, l_ref = _textbook_attention(q[0, h], k[0, h], v[0, h], scale)
        assert np.allclose(res["o"][0, h], o_ref, rtol=0, atol=1e-13)
        assert np.allclose(res["lse"][0, h], l_ref, rtol=0, atol=1e-13)
    # library routine (torch CPU fp64 scaled_dot_product_attention), larger
    B, H, Nq, Nk, D, b = 2, 3, 300, 517, 64, 128
    q = rng.standard_normal((B, H, Nq, D))
    k = rng.standard_normal((B, H, Nk, D))
    v = rng.standard_normal((B, H, Nk, D))
    res = impl.run_pipeline(q, k, v, n_forced_tokens=128, density=1.0, block=b)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                         torch.from_numpy(v)).numpy()
    assert np.abs(res["o"] - ref).max() <= 1e-12
    lse_ref = logsumexp(np.einsum("bhqd,bhkd->bhqk", q, k) / math.sqrt(D), axis=-1)
    assert np.abs(res["lse"] - lse_ref).max() <= 1e-12


def pin_masked_sdpa(impl, seed=5):
    """At any density, equal to dense attention with a boolean mask that
    admits exactly the keys of the kept blocks."""
    rng = np.random.default_rng(seed)
    B, H, Nq, Nk, D, b = 1, 2, 700, 1000, 32, 128
    q = rng.standard_normal((B, H, Nq, D))
    k = rng.standard_normal((B, H, Nk, D)) + rng.standard_normal((B, H, 1, D))
    v = rng.standard_normal((B, H, Nk, D))
    for dens in (0.25, 0.5, 0.09375):
        res = impl.run_pipeline(q, k, v, n_forced_tokens=130, density=dens, block=b)
        mask = np.zeros((B, H, Nq, Nk), dtype=bool)
        for h in range(H):
            for i in range(-(-Nq // b)):
                for j in res["kv_index"][0, h, i, :res["kv_count"][0, h, i]]:
                    mask[0, h, i * b:(i + 1) * b, j * b:(j + 1) * b] = True
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v),
                                             attn_mask=torch.from_numpy(mask)).numpy()
        assert np.abs(res["o"] - ref).max() <= 1e-12, dens
        logits = np.where(mask, np.einsum("bhqd,bhkd->bhqk", q, k) / math.sqrt(D), -np.inf)
        assert np.abs(res["lse"] - logsumexp(logits, axis=-1)).max() <= 1e-12


def pin_convex_hull(impl, seed=6):
    """Each output is a convex combination of the kept value rows."""
    rng = np.random.default_rng(seed)
    B, H, Nq, Nk, D, b = 1, 1, 256, 640, 16, 128
    q = rng.standard_normal((B, H, Nq, D)) * 3
    k = rng.standard_normal((B, H, Nk, D))
    v = rng.standard_normal((B, H, Nk, D))
    res = impl.run_pipeline(q, k, v, n_forced_tokens=0, density=0.5, block=b)
    for i in range(2):
        blocks = res["kv_index"][0, 0, i, :res["kv_count"][0, 0, i]]
        keys = np.concatenate([np.arange(j * b, min((j + 1) * b, Nk)) for j in blocks])
        vs = v[0, 0, keys]
        o = res["o"][0, 0, i * b:(i + 1) * b]
        assert np.all(o <= vs.max(axis=0) + 1e-12) and np.all(o >= vs.min(axis=0) - 1e-12)


def pin_empty_selection(impl):
    """Nothing forced and density 0: no key is kept, O = 0, LSE = -inf."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 130, 8))
    k = rng.standard_normal((1, 1, 300, 8))
    v = rng.standard_normal((1, 1, 300, 8))
    res = impl.run_pipeline(q, k, v, n_forced_tokens=0, density=0.0, block=128)
    assert np.all(res["kv_count"] == 0)
    assert np.all(res["kv_index"] == -1) or res["kv_index"].shape[-1] == 0
    assert np.all(res["o"] == 0) and np.all(np.isneginf(res["lse"]))


def pin_selected_flops(impl):
    """Closed form: with full blocks, 4 * D * Nq * kept * b."""
    B, H, nqb, kept, D, b = 1, 2, 3, 5, 64, 128
    count = np.full((B, H, nqb), kept, dtype=np.int32)
    index = np.tile(np.arange(kept, dtype=np.int32), (B, H, nqb, 1))
    assert impl.selected_flops(count, index, nqb * b, 10 * b, D, b) == 4 * D * (nqb * b) * kept * b * B * H
    # partial last query block (10 tokens) and partial last key block (5 tokens)
    index2 = np.tile(np.array([0, 9], dtype=np.int32), (1, 1, 1, 1))
    count2 = np.array([[[2]]], dtype=np.int32)
    assert impl.selected_flops(count2, index2, 10, 9 * b + 5, D, b) == 4 * D * 10 * (b + 5)


# --- retained attention mass and the token-wise Top-K bound -------------------
def _textbook_probs(q, k, scale):
    """Dense softmax probabilities, one query at a time with exact sums."""
    out = []
    for t in range(q.shape[0]):
        logits = [scale * math.fsum(q[t, d] * k[s, d] for d in range(q.shape[1]))
                  for s in range(k.shape[0])]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = math.fsum(w)
        out.append([x / z for x in w])
    return out


def pin_retained_mass(impl, seed=8):
    """Retained mass = dense softmax probability summed over the kept keys
    ([R] 'Core claim'): brute force on tiny inputs; exactly 1 when every block
    is kept; never decreasing as the density grows (top-k sets are nested);
    equal to exp(LSE over kept keys - LSE over all keys)."""
    rng = np.random.default_rng(seed)
    B, H, Nq, Nk, D, b = 1, 1, 6, 13, 4, 4
    q = rng.standard_normal((B, H, Nq, D)) * 2
    k = rng.standard_normal((B, H, Nk, D))
    v = rng.standard_normal((B, H, Nk, D))
    res = impl.run_pipeline(q, k, v, n_forced_tokens=3, density=0.34, block=b)
    rows = [(0, 0, i) for i in range(-(-Nq // b))]
    got = impl.retained_mass_rows(q, k, res["kv_count"], res["kv_index"], rows, block=b)
    scale = 1 / math.sqrt(D)
    for (_, _, i) in rows:
        qb = q[0, 0, i * b:min((i + 1) * b, Nq)]
        probs = _textbook_probs(qb, k[0, 0], scale)
        blocks = list(res["kv_index"][0, 0, i, :res["kv_count"][0, 0, i]])
        for t, pr in enumerate(probs):
            ref = math.fsum(pr[s] for s in range(Nk) if s // b in blocks)
            assert abs(got[(0, 0, i)][t] - ref) <= 1e-13, (i, t)
    # density 1 keeps everything; nesting over densities; LSE identity
    B, H, Nq, Nk, D, b = 1, 2, 300, 700, 16, 128
    q = rng.standard_normal((B, H, Nq, D)) * 2
    k = rng.standard_normal((B, H, Nk, D)) + rng.standard_normal((B, H, 1, D))
    v = rng.standard_normal((B, H, Nk, D))
    rows = [(0, h, i) for h in range(H) for i in range(-(-Nq // b))]
    prev = None
    full = impl.run_pipeline(q, k, v, n_forced_tokens=0, density=1.0, block=b)
    for dens in (0.0, 0.2, 0.4, 0.6, 1.0):
        res = impl.run_pipeline(q, k, v, n_forced_tokens=130, density=dens, block=b)
        m = impl.retained_mass_rows(q, k, res["kv_count"], res["kv_index"], rows, block=b)
        cur = np.concatenate([m[r] for r in rows])
        assert np.all(cur > 0) and np.all(cur <= 1 + 1e-12)
        if prev is not None:
            assert np.all(cur >= prev - 1e-12), dens
        for (bb, h, i) in rows:
            lo = i * b
            hi = lo + m[(bb, h, i)].size
            ident = np.exp(res["lse"][bb, h, lo:hi] - full["lse"][bb, h, lo:hi])
            assert np.abs(m[(bb, h, i)] - ident).max() <= 1e-12
        prev = cur
    assert np.abs(prev - 1).max() <= 1e-12


def pin_token_topk_bound(impl, seed=9):
    """The token-wise Top-K policy at the same budget keeps the forced tokens
    and the k * b most probable eligible keys per query ([R] 'Core claim',
    'Editorial extensions'): brute force by ranking probabilities on tiny
    inputs; never below the block policy's retained mass; 1 when every
    eligible key fits the budget; the forced mass alone when the budget is 0."""
    rng = np.random.default_rng(seed)
    B, H, Nq, Nk, D, b = 1, 1, 5, 14, 4, 4
    q = rng.standard_normal((B, H, Nq, D)) * 2
    k = rng.standard_normal((B, H, Nk, D))
    scale = 1 / math.sqrt(D)
    F, kb = 1, 2
    rows = [(0, 0, i) for i in range(-(-Nq // b))]
    got = impl.token_topk_bound_rows(q, k, F, kb, rows, block=b)
    for (_, _, i) in rows:
        qb = q[0, 0, i * b:min((i + 1) * b, Nq)]
        for t, pr in enumerate(_textbook_probs(qb, k[0, 0], scale)):
            elig = sorted(pr[F * b:], reverse=True)
            ref = math.fsum(pr[:F * b]) + math.fsum(elig[:kb * b])
            assert abs(got[(0, 0, i)][t] - ref) <= 1e-13, (i, t)
    B, H, Nq, Nk, D, b = 1, 2, 300, 700, 16, 128
    q = rng.standard_normal((B, H, Nq, D)) * 2
    k = rng.standard_normal((B, H, Nk, D)) + rng.standard_normal((B, H, 1, D))
    v = rng.standard_normal((B, H, Nk, D))
    rows = [(0, h, i) for h in range(H) for i in range(-(-Nq // b))]
    for dens in (0.0, 0.25, 0.5):
        res = impl.run_pipeline(q, k, v, n_forced_tokens=130, density=dens, block=b, attention=False)
        F = res["n_forced"]
        kblk = int(res["kv_count"][0, 0, 0]) - F
        m = impl.retained_mass_rows(q, k, res["kv_count"], res["kv_index"], rows, block=b)
        u = impl.token_topk_bound_rows(q, k, F, kblk, rows, block=b)
        for r in rows:
            assert np.all(u[r] >= m[r] - 1e-12), (dens, r)
            if kblk == 0:
                assert np.abs(u[r] - m[r]).max() <= 1e-12
    nkb = -(-700 // 128)
    u = impl.token_topk_bound_rows(q, k, 2, nkb - 2, rows, block=128)
    assert all(np.abs(u[r] - 1).max() <= 1e-12 for r in rows)


# --- mask reuse: block maps between scales ----------------------------------
def pin_transfer_golden(impl):
    """Block maps worked by hand from the mask-reuse reading (tests/golden/
    transfer_tiny.json): upsampling, downsampling, a partial last block and a
    block straddling two segments."""
    g = _golden("transfer_tiny.json")
    for c in g["cases"]:
        km = impl.transfer_key_map(c["src"], c["dst"], c["block"])
        qm = impl.transfer_query_map(c["src"][2], c["dst"][2], c["block"])
        assert km.tolist() == c["key_map"], (c["note"], km.tolist())
        assert qm.tolist() == c["query_map"], (c["note"], qm.tolist())


def pin_transfer_identity(impl, seed=10):
    """The same geometry on both sides maps every block to itself, so the
    reused scores are the source scores and the reused selection is the
    fresh one (any geometry, partial blocks and straddling blocks included)."""
    rng = np.random.default_rng(seed)
    for geom in [(0, 0, 300), (512, 0, 1000), (512, 3600, 7000), (100, 200, 50), (1, 1, 1)]:
        for b in (32, 128):
            n = sum(geom)
            assert impl.transfer_key_map(geom, geom, b).tolist() == list(range(-(-n // b)))
            assert impl.transfer_query_map(geom[2], geom[2], b).tolist() == list(range(-(-geom[2] // b)))
    geom = (512, 1000, 1300)
    S = rng.standard_normal((2, 3, -(-1300 // 128), -(-2812 // 128)))
    T = impl.transfer_scores(S, geom, geom)
    assert np.array_equal(T, S)
    c1, i1 = impl.transferred_selection(S, geom, geom, 4, 0.25)
    c2, i2 = impl.select_blocks(S, 4, 0.25)
    assert np.array_equal(c1, c2) and np.array_equal(i1, i2)


def pin_transfer_integer_upsample(impl):
    """Block-aligned segments scaled by an integer factor m: every source block
    of a scaled segment is reused by exactly m consecutive target blocks (a
    closed form), the unscaled text segment maps to itself."""
    b = 128
    for m in (2, 3):
        src = (256, 3 * b, 5 * b)
        dst = (256, 3 * b * m, 5 * b * m)
        km = impl.transfer_key_map(src, dst, b)
        expect = [0, 1] + [2 + j // m for j in range(3 * m)] + [5 + j // m for j in range(5 * m)]
        assert km.tolist() == expect, (m, km.tolist())
        qm = impl.transfer_query_map(src[2], dst[2], b)
        assert qm.tolist() == [j // m for j in range(5 * m)]
        # the other way round every m-th source block is taken: block m*j + m//2
        km_down = impl.transfer_key_map(dst, src, b)
        assert km_down.tolist() == [0, 1] + [2 + m * j + m // 2 for j in range(3)] + \
            [2 + 3 * m + m * j + m // 2 for j in range(5)], (m, km_down.tolist())


def pin_transfer_invariants(impl, seed=11):
    """Random geometries: maps stay in range, never decrease, and the source
    token they land on lies in the same segment as the target block's centre
    (checked here by a direct scan over tokens, not by the map's arithmetic)."""
    rng = np.random.default_rng(seed)
    for _ in range(40):
        b = int(rng.choice([4, 32, 128]))
        t = int(rng.integers(0, 300))
        src = (t, int(rng.integers(1, 2000)), int(rng.integers(1, 2000)))
        dst = (t, int(rng.integers(1, 2000)), int(rng.integers(1, 2000)))
        km = impl.transfer_key_map(src, dst, b)
        qm = impl.transfer_query_map(src[2], dst[2], b)
        assert km.size == -(-sum(dst) // b) and qm.size == -(-dst[2] // b)
        assert km.min() >= 0 and km.max() < -(-sum(src) // b)
        assert qm.min() >= 0 and qm.max() < -(-src[2] // b)
        assert np.all(np.diff(km) >= 0) and np.all(np.diff(qm) >= 0)
        seg_src = np.repeat([0, 1, 2], src)
        seg_dst = np.repeat([0, 1, 2], dst)
        n_dst = sum(dst)
        for j in range(km.size):
            lo, hi = j * b, min((j + 1) * b, n_dst)
            # centre of [lo, hi) is (lo + hi) / 2: the token holding it
            seg = seg_dst[(lo + hi) // 2] if (lo + hi) % 2 == 0 else seg_dst[(lo + hi - 1) // 2]
            toks = np.arange(km[j] * b, min((km[j] + 1) * b, sum(src)))
            assert np.any(seg_src[toks] == seg), (src, dst, b, j)
    try:
        impl.transfer_key_map((0, 0, 100), (0, 50, 100), 32)
    except ValueError:
        pass
    else:
        raise AssertionError("a target segment with no source counterpart must be refused")


ALL_PINS = [pin_identity, pin_means_closed_form, pin_selection_bruteforce,
            pin_ties_duplicated_blocks, pin_tiny_budget, pin_dense_equivalence,
            pin_masked_sdpa, pin_convex_hull, pin_empty_selection, pin_selected_flops,
            pin_retained_mass, pin_token_topk_bound, pin_transfer_golden,
            pin_transfer_identity, pin_transfer_integer_upsample, pin_transfer_invariants]
