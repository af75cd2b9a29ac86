"""GPU parity, stage by stage, on seeded inputs that span several tiles and a
ragged tail.  Every call goes through the C ABI (ctypes binding)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_head_amd as sp
import oracle
from tests.parity_util import (check_selection, compare_lse, compare_outputs, log, to_dev,
                               to_f64)
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu


def _rand(shape, dtype, seed, offset=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32) + np.float32(offset)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


# ---------------------------------------------------------------- block means
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 127, 128, 1000, 1280])
def test_block_means(dtype, D, N):
    log(f"means dtype={dtype} D={D} N={N}")
    x = _rand((2, 3, N, D), dtype, seed=N + D, offset=0.3)
    g = to_f64(sp.block_means(to_dev(x, dtype)))
    ref = oracle.block_means(oracle.decode(x, dtype))
    assert g.shape == ref.shape
    # fp32 rounding of a nearly exact mean: within 2 ulp of the float64 value
    err = np.abs(g - ref)
    assert np.all(err <= 2.0 ** -22 * np.abs(ref) + 1e-30), float((err / np.abs(ref)).max())


# ---------------------------------------------------------------- block scores
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("nqb,nkb", [(1, 1), (16, 16), (70, 131), (141, 286)])
def test_block_scores(D, nqb, nkb):
    log(f"scores D={D} nqb={nqb} nkb={nkb}")
    rng = np.random.default_rng(nqb * 1000 + nkb)
    qb = (rng.standard_normal((2, 2, nqb, D)) * 0.3).astype(np.float32)
    kb = (rng.standard_normal((2, 2, nkb, D)) * 0.3).astype(np.float32)
    tau = 1.0 / math.sqrt(D)
    g = to_f64(sp.block_scores(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda()))
    ref = oracle.block_scores(qb.astype(np.float64), kb.astype(np.float64))
    # float64 accumulation rounded once: within 1 ulp of the float32 value, plus
    # the float32 rounding of tau (a common factor for every score)
    err = np.abs(g - ref)
    bound = 2.0 ** -22 * np.abs(ref) + 1e-9 * np.abs(ref).max()
    assert np.all(err <= bound), float(err.max())


# ---------------------------------------------------------------- selection
SEL_CASES = [
    # nkb, F, density, kind
    (16, 1, 0.25, "normal"), (286, 4, 0.1875, "normal"), (1129, 4, 0.09375, "normal"),
    (595, 33, 0.09375, "normal"), (129, 4, 0.625, "ties"), (300, 0, 0.5, "nan"),
    (200, 10, 1.0, "normal"), (64, 0, 0.0, "normal"), (65, 65, 0.5, "normal"),
    (2048, 4, 0.09375, "ties"), (2100, 4, 0.1, "normal"), (3000, 7, 0.3, "nan"),
    (1, 0, 1.0, "normal"), (500, 3, 0.2, "inf"), (257, 2, 0.33, "zeros"),
    (2300, 4, 0.09375, "normal"), (4516, 4, 0.09375, "ties"), (4700, 9, 0.2, "nan"),
]


@pytest.mark.parametrize("nkb,F,density,kind", SEL_CASES)
def test_select_blocks(nkb, F, density, kind):
    log(f"select nkb={nkb} F={F} density={density} kind={kind}")
    rng = np.random.default_rng(nkb + F)
    B, H, nqb = 1, 3, 37
    S = rng.standard_normal((B, H, nqb, nkb)).astype(np.float32)
    if kind == "ties":
        S = (np.round(S * 4) / 4).astype(np.float32)
    elif kind == "nan":
        S[rng.random(S.shape) < 0.3] = np.nan
    elif kind == "inf":
        S[rng.random(S.shape) < 0.05] = np.inf
        S[rng.random(S.shape) < 0.05] = -np.inf
    elif kind == "zeros":
        S[rng.random(S.shape) < 0.5] = 0.0
        S[rng.random(S.shape) < 0.5] = -0.0
    kept = sp.kept_blocks(nkb, F, density)
    max_kept = kept + 3   # padding must be written as -1
    cnt, idx = sp.select_blocks(torch.from_numpy(S).cuda(), F, density, max_kept=max_kept)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    o_cnt, o_idx = oracle.select_blocks(S.astype(np.float64), F, density, max_kept=max_kept)
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(idx, o_idx)


# ------------------------------------------------- fused scores + selection
FUSED_CASES = [
    # D, nqb, nkb, F, density, kind
    (128, 1, 1, 0, 1.0, "normal"), (128, 16, 16, 1, 0.25, "normal"),
    (128, 37, 131, 4, 0.1875, "normal"), (64, 70, 286, 4, 0.1875, "normal"),
    (128, 17, 567, 33, 0.09375, "normal"), (64, 33, 1129, 4, 0.09375, "normal"),
    (128, 5, 2048, 4, 0.09375, "normal"), (128, 40, 300, 0, 0.5, "ties"),
    (64, 21, 129, 4, 0.625, "ties"), (128, 9, 200, 10, 0.0, "normal"),
    (128, 9, 65, 65, 0.5, "normal"), (64, 3, 1000, 2, 1.0, "ties"),
    # groups of near-duplicate key blocks: bands of a few blocks decided on
    # exact scores, and larger groups that exceed the band capacity
    (128, 37, 1129, 4, 0.09375, "near"), (64, 40, 600, 3, 0.25, "near"),
    (128, 20, 2048, 4, 0.1875, "near_wide"), (128, 33, 1129, 4, 0.09375, "scaled"),
    (128, 18, 300, 4, 0.5, "neg_tau"), (128, 18, 300, 4, 0.5, "zero_tau"),
    (64, 17, 700, 0, 0.0, "normal"), (128, 21, 1500, 1500, 0.3, "normal"),
]


def _fused_means(D, nqb, nkb, kind, seed):
    rng = np.random.default_rng(seed)
    qb = (rng.standard_normal((2, 2, nqb, D)) * 0.3).astype(np.float32)
    kb = (rng.standard_normal((2, 2, nkb, D)) * 0.3).astype(np.float32)
    if kind in ("near", "near_wide"):
        # every key block is one of few base vectors plus a relative
        # perturbation of ~1e-6 (near) or ~1e-7 (near_wide): the scores come
        # in tight clusters of 6 (near) or 40 (near_wide) blocks
        g = 6 if kind == "near" else 40
        base = kb[:, :, ::g].repeat(g, axis=2)[:, :, :nkb]
        eps = 1e-6 if kind == "near" else 1e-7
        kb = (base * (1 + eps * rng.standard_normal(base.shape))).astype(np.float32)
    elif kind == "scaled":
        # means far from unit scale (the bound scales with them)
        qb = (qb * 3e3).astype(np.float32)
        kb = (kb * 2e-3).astype(np.float32)
    if kind == "ties":
        # few distinct small dyadic values: many scores are exactly equal
        # (dyadic values: every score is exact, distinct sums stay far apart)
        qb = (np.round(qb * 4) / 4).astype(np.float32)
        kb = np.round(kb * 2).clip(-1, 1).astype(np.float32)
        kb[:, :, 1::2] = kb[:, :, 0:nkb - 1:2]     # duplicated key blocks tie exactly
    return qb, kb


@pytest.mark.parametrize("D,nqb,nkb,F,density,kind", FUSED_CASES)
def test_fused_select_matches_two_step(D, nqb, nkb, F, density, kind):
    log(f"fused select D={D} nqb={nqb} nkb={nkb} F={F} density={density} kind={kind}")
    qb, kb = _fused_means(D, nqb, nkb, kind, seed=nqb * 7 + nkb)
    q_t, k_t = torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda()
    tau = {"neg_tau": -1.0 / math.sqrt(D), "zero_tau": 0.0}.get(kind, 1.0 / math.sqrt(D))
    max_kept = sp.kept_blocks(nkb, F, density) + 2
    c1, i1 = sp.select_blocks_from_means(q_t, k_t, F, density, tau=tau, max_kept=max_kept)
    S = sp.block_scores(q_t, k_t, tau=tau)
    c2, i2 = sp.select_blocks(S, F, density, max_kept=max_kept)
    c1, i1, c2, i2 = (t.cpu().numpy() for t in (c1, i1, c2, i2))
    # same scores, same rule: identical to the two-call route
    assert np.array_equal(c1, c2)
    assert np.array_equal(i1, i2)
    # and the oracle's selection up to the near-tie rule
    ref_S = oracle.block_scores(qb.astype(np.float64), kb.astype(np.float64), tau=tau)
    swaps = check_selection(ref_S, F, density, c1, i1)
    log(f"  {c1.size} rows, {swaps} near-tie swaps")
    if kind == "ties":
        # exact ties in float64 stay exact ties in float32: no swap allowed
        assert swaps == 0


def test_fused_select_repeated_calls_share_nothing():
    # two launches in a row on different shapes: the second is not affected by the first
    qb, kb = _fused_means(128, 30, 700, "normal", seed=5)
    c_a, i_a = sp.select_blocks_from_means(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(),
                                           4, 0.1)
    qs, ks = qb[:1, :1, :3], kb[:1, :1, :50]
    c_b, i_b = sp.select_blocks_from_means(torch.from_numpy(np.ascontiguousarray(qs)).cuda(),
                                           torch.from_numpy(np.ascontiguousarray(ks)).cuda(), 4, 0.1)
    for (qq, kk, c, i) in ((qb, kb, c_a, i_a), (qs, ks, c_b, i_b)):
        ref_S = oracle.block_scores(qq.astype(np.float64), kk.astype(np.float64))
        check_selection(ref_S, 4, 0.1, c.cpu().numpy(), i.cpu().numpy())


QK_CASES = [
    # dtype, D, block, Nq, Nk, F, density
    ("bf16", 128, 128, 1000, 3000, 4, 0.25), ("fp32", 64, 64, 333, 2049, 0, 0.5),
    ("bf16", 64, 32, 129, 4500, 2, 0.125), ("fp32", 128, 128, 1, 1, 0, 1.0),
    ("bf16", 128, 128, 5000, 131000, 4, 0.09375), ("bf16", 128, 64, 777, 20000, 40, 0.0),
]


@pytest.mark.parametrize("dtype,D,block,Nq,Nk,F,density", QK_CASES)
def test_select_from_qk_matches_the_separate_calls(dtype, D, block, Nq, Nk, F, density):
    """One call for the whole selection stage (means of Q and K, then the
    screened route) equals the means calls and select_blocks_from_means bit
    for bit, means included."""
    log(f"select from qk dtype={dtype} D={D} block={block} Nq={Nq} Nk={Nk} F={F} density={density}")
    B, H = 1, 2
    q = to_dev(_rand((B, H, Nq, D), dtype, seed=Nq + 3, offset=0.1), dtype)
    k = to_dev(_rand((B, H, Nk, D), dtype, seed=Nk + 5, offset=0.2), dtype)
    c1, i1, qb1, kb1 = sp.select_blocks_from_qk(q, k, F, density, block=block)
    qb2, kb2 = sp.block_means(q, block), sp.block_means(k, block)
    c2, i2 = sp.select_blocks_from_means(qb2, kb2, F, density)
    assert torch.equal(qb1, qb2) and torch.equal(kb1, kb2)
    assert torch.equal(c1, c2) and torch.equal(i1, i2)
    # and the selection is the oracle's on the kernel's own means
    S = oracle.block_scores(to_f64(qb1), to_f64(kb1))
    check_selection(S, F, density, c1.cpu().numpy(), i1.cpu().numpy())


# ---------------------------------------------------------------- attention
def _attn_case(dtype, D, Nq, Nk, density, F_tokens, seed):
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    q = rng.standard_normal((B, H, Nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    nkb = -(-Nk // 128)
    k += rng.standard_normal((B, H, nkb, 1, D), dtype=np.float32).repeat(128, axis=3).reshape(
        B, H, nkb * 128, D)[:, :, :Nk] * np.float32(0.5)
    if dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    qd, kd, vd = (oracle.decode(a, dtype) for a in (q, k, v))
    res = oracle.run_pipeline(qd, kd, vd, F_tokens, density, attention=False)
    return (q, k, v), (qd, kd, vd), res


def _check_attn(dtype, q, k, v, qd, kd, vd, cnt, idx, what):
    cnt_t = torch.from_numpy(np.ascontiguousarray(cnt, dtype=np.int32)).cuda()
    idx_t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    o, lse = sp.block_sparse_attn_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                      cnt_t, idx_t)
    # the oracle skips nothing, so hand it the valid entries only
    nkb = -(-kd.shape[2] // 128)
    rows = cnt.size
    clean_cnt = np.zeros_like(cnt)
    clean_idx = np.full_like(idx, -1)
    flat_c, flat_i = clean_cnt.reshape(-1), clean_idx.reshape(rows, -1)
    src_c, src_i = cnt.reshape(-1), idx.reshape(rows, -1)
    for r in range(rows):
        row = [j for j in src_i[r, :max(0, min(src_c[r], src_i.shape[1]))] if 0 <= j < nkb]
        flat_c[r] = len(row)
        flat_i[r, :len(row)] = row
    o_ref, lse_ref = oracle.sparse_attention(qd, kd, vd, clean_cnt, clean_idx)
    mx, rel = compare_outputs(to_f64(o), o_ref, dtype, what)
    compare_lse(to_f64(lse), lse_ref, 1e-4 if dtype == "fp32" else 2e-3, what)
    log(f"  {what}: max|dO|={mx:.3g} relL2={rel}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nk,density,F_tokens", [
    (300, 1000, 0.5, 130), (128, 2048, 0.25, 128), (1, 129, 1.0, 0), (700, 777, 0.0, 200),
])
def test_attention(dtype, D, Nq, Nk, density, F_tokens):
    log(f"attn dtype={dtype} D={D} Nq={Nq} Nk={Nk} density={density} F={F_tokens}")
    (q, k, v), (qd, kd, vd), res = _attn_case(dtype, D, Nq, Nk, density, F_tokens, seed=Nq + Nk)
    _check_attn(dtype, q, k, v, qd, kd, vd, res["kv_count"], res["kv_index"], "oracle index")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_attention_index_edge_cases(dtype):
    """Empty rows, out-of-range entries (skipped), counts beyond max_kept
    (clamped), a permuted list, and the dense list."""
    log(f"attn edge cases dtype={dtype}")
    Nq, Nk = 520, 1100
    (q, k, v), (qd, kd, vd), res = _attn_case(dtype, 128, Nq, Nk, 0.5, 0, seed=11)
    cnt, idx = res["kv_count"].copy(), res["kv_index"].copy()
    nkb = 9
    idx = np.concatenate([idx, np.full(idx.shape[:-1] + (nkb + 1 - idx.shape[-1],), -1, np.int32)],
                         axis=-1)
    cnt[0, 0, 0] = 0                                  # empty row -> O = 0, LSE = -inf
    idx[0, 0, 1, 1] = nkb + 5                         # out of range -> skipped
    idx[0, 0, 2, 0] = -7                              # negative -> skipped
    cnt[0, 1, 0] = idx.shape[-1] + 10                 # clamped to max_kept
    idx[0, 1, 0, :] = -1
    idx[0, 1, 0, :3] = [8, 0, 4]                      # permuted order, includes partial block
    idx[0, 1, 1, :nkb] = np.arange(nkb)[::-1]         # dense, reversed
    cnt[0, 1, 1] = nkb
    _check_attn(dtype, q, k, v, qd, kd, vd, cnt, idx, "edge cases")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_attention_order_invariance(dtype):
    """Permuting each index list changes only the summation order."""
    log(f"attn order invariance dtype={dtype}")
    (q, k, v), (qd, kd, vd), res = _attn_case(dtype, 128, 640, 1500, 0.4, 256, seed=5)
    cnt, idx = res["kv_count"], res["kv_index"].copy()
    rng = np.random.default_rng(0)
    for r in np.ndindex(cnt.shape):
        c = cnt[r]
        idx[r][:c] = rng.permutation(idx[r][:c])
    _check_attn(dtype, q, k, v, qd, kd, vd, cnt, idx, "permuted")


def test_selection_feeds_attention_dense_equivalence():
    """At density 1 the GPU path equals dense softmax attention."""
    log("dense equivalence through the whole GPU path")
    (q, k, v), (qd, kd, vd), _ = _attn_case("bf16", 128, 384, 900, 1.0, 0, seed=3)
    out = sp.sparse_attention(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), 0, 1.0,
                              return_all=True)
    assert np.all(out["kv_count"].cpu().numpy() == 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(vd)).numpy()
    compare_outputs(to_f64(out["o"]), ref, "bf16", "dense")


# ------------------------------------------------------ retained attention mass
@pytest.mark.parametrize("dtype,D,Nq,Nk,density,F_tokens", [
    ("fp32", 64, 700, 1500, 0.25, 128), ("bf16", 128, 1000, 2400, 0.1875, 300),
    ("bf16", 64, 513, 1100, 0.5, 0),
])
def test_retained_mass(dtype, D, Nq, Nk, density, F_tokens):
    log(f"retained mass dtype={dtype} D={D} Nq={Nq} Nk={Nk} density={density}")
    (q, k, v), (qd, kd, vd), res = _attn_case(dtype, D, Nq, Nk, density, F_tokens, seed=Nq + Nk)
    cnt, idx = res["kv_count"], res["kv_index"]
    g = sp.selection_retained_mass(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                   torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    g = to_f64(g)
    B, H = cnt.shape[:2]
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(cnt.shape[2])]
    ref = oracle.retained_mass_rows(qd, kd, cnt, idx, rows)
    tol = 1e-5 if dtype == "fp32" else 5e-3   # from the LSE tolerances of the two attention calls
    worst = 0.0
    for (b, h, i), m in ref.items():
        got = g[b, h, i * 128:i * 128 + m.size]
        worst = max(worst, float(np.abs(got - m).max()))
    log(f"  max |mass - oracle| = {worst:.3g}")
    assert worst <= tol


def test_retained_mass_full_selection_is_one():
    # every block kept: both LSEs come from identical lists, so the mass is exactly 1
    (q, k, v), _, res = _attn_case("bf16", 128, 600, 900, 1.0, 0, seed=3)
    g = sp.selection_retained_mass(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                   torch.from_numpy(res["kv_count"]).cuda(),
                                   torch.from_numpy(res["kv_index"]).cuda())
    assert torch.all(g == 1.0)


def test_retained_mass_edge_values():
    lse_s = torch.tensor([0.0, -float("inf"), 1.5, -2.0, 3.0], device="cuda")
    lse_d = torch.tensor([0.0, 0.0, 2.0, -float("inf"), 3.0 + math.log(4.0)], device="cuda")
    m = sp.retained_mass(lse_s, lse_d).cpu().numpy()
    ref = np.array([1.0, 0.0, math.exp(-0.5), 0.0, 0.25])
    assert np.allclose(m, ref, rtol=2e-7, atol=0)


# ------------------------------------------------------------- graph capture
def test_scale_captured_in_a_graph():
    """The whole scale (two means, scores, selection, attention) recorded as one
    HIP graph and replayed: every replay equals the eager result bit for bit,
    with eager work and synchronisations between replays."""
    (q, k, v), _, res = _attn_case("bf16", 128, 1100, 2600, 0.1875, 300, seed=11)
    qd, kd, vd = (to_dev(a, "bf16") for a in (q, k, v))
    B, H, Nq, D = qd.shape
    nqb, nkb = -(-Nq // 128), -(-kd.shape[2] // 128)
    F = sp.forced_blocks(300)
    kept = sp.kept_blocks(nkb, F, 0.1875)
    f32, i32, dev = torch.float32, torch.int32, qd.device
    bufs = {"qbar": torch.empty((B, H, nqb, D), dtype=f32, device=dev),
            "kbar": torch.empty((B, H, nkb, D), dtype=f32, device=dev),
            "S": torch.empty((B, H, nqb, nkb), dtype=f32, device=dev),
            "cnt": torch.empty((B, H, nqb), dtype=i32, device=dev),
            "idx": torch.empty((B, H, nqb, kept), dtype=i32, device=dev),
            "o": torch.empty_like(qd), "lse": torch.empty((B, H, Nq), dtype=f32, device=dev)}

    def scale():
        sp.block_means(qd, out=bufs["qbar"])
        sp.block_means(kd, out=bufs["kbar"])
        sp.block_scores(bufs["qbar"], bufs["kbar"], out=bufs["S"])
        sp.select_blocks(bufs["S"], F, 0.1875, max_kept=kept, kv_count=bufs["cnt"],
                         kv_index=bufs["idx"])
        sp.block_sparse_attn_fwd(qd, kd, vd, bufs["cnt"], bufs["idx"], out=bufs["o"],
                                 lse=bufs["lse"])

    scale()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in bufs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream once
        scale()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        scale()
    for rep in range(3):
        for t in bufs.values():
            t.zero_()                       # replays must rewrite everything
        g.replay()
        torch.cuda.synchronize()
        for n, t in bufs.items():
            assert torch.equal(t, eager[n]), (rep, n)
        scale()                             # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("route", ["from_qk", "noalloc"])
def test_screened_scale_captured_in_a_graph(route):
    """The scale on the screened route recorded as one HIP graph: the
    whole-stage call with a caller workspace, or the means and the
    allocation-free selection (the entry point meant for capture); every
    replay equals the eager result bit for bit, with eager work between."""
    (q, k, v), _, res = _attn_case("bf16", 128, 1100, 2600, 0.1875, 300, seed=12)
    qd, kd, vd = (to_dev(a, "bf16") for a in (q, k, v))
    B, H, Nq, D = qd.shape
    nqb, nkb = -(-Nq // 128), -(-kd.shape[2] // 128)
    F = sp.forced_blocks(300)
    kept = sp.kept_blocks(nkb, F, 0.1875)
    f32, i32, dev = torch.float32, torch.int32, qd.device
    bufs = {"qbar": torch.empty((B, H, nqb, D), dtype=f32, device=dev),
            "kbar": torch.empty((B, H, nkb, D), dtype=f32, device=dev),
            "cnt": torch.empty((B, H, nqb), dtype=i32, device=dev),
            "idx": torch.empty((B, H, nqb, kept), dtype=i32, device=dev),
            "o": torch.empty_like(qd), "lse": torch.empty((B, H, Nq), dtype=f32, device=dev)}
    ws = sp.select_workspace(B, H, nqb, nkb, dev)

    def scale():
        if route == "from_qk":
            sp.select_blocks_from_qk(qd, kd, F, 0.1875, max_kept=kept, qbar=bufs["qbar"],
                                     kbar=bufs["kbar"], kv_count=bufs["cnt"],
                                     kv_index=bufs["idx"], workspace=ws)
        else:
            sp.block_means(qd, out=bufs["qbar"])
            sp.block_means(kd, out=bufs["kbar"])
            sp.select_blocks_from_means_noalloc(bufs["qbar"], bufs["kbar"], F, 0.1875,
                                                max_kept=kept, kv_count=bufs["cnt"],
                                                kv_index=bufs["idx"])
        sp.block_sparse_attn_fwd(qd, kd, vd, bufs["cnt"], bufs["idx"], out=bufs["o"],
                                 lse=bufs["lse"])

    scale()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in bufs.items()}
    # the screened route selects what the two-call route selects
    c2, i2 = sp.select_blocks(sp.block_scores(eager["qbar"], eager["kbar"]), F, 0.1875,
                              max_kept=kept)
    assert torch.equal(c2, eager["cnt"]) and torch.equal(i2, eager["idx"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm the capture stream once
        scale()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        scale()
    for rep in range(3):
        for t in bufs.values():
            t.zero_()                       # replays must rewrite everything
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        for n, t in bufs.items():
            assert torch.equal(t, eager[n]), (route, rep, n)
        scale()                             # eager work between replays
        torch.cuda.synchronize()
