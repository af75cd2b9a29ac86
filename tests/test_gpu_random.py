"""GPU parity of the whole path on seeded random shapes: batch, heads, head
size, dtype, block size, ragged sequence lengths, forced prefixes and
densities drawn at random (all valid), every row checked against the oracle.
Complements the fixed workloads with shapes nobody picked by hand."""
import numpy as np
import pytest

import block_sparse_attention_head_amd as sp
import oracle
from tests.parity_util import check_selection, compare_lse, compare_outputs, log, to_dev, to_f64
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

DENSITIES = (0.0, 0.0625, 0.1875, 0.25, 0.5, 1.0)   # dyadic, as the pages' schedule


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "fp32" if seed % 7 == 3 else "bf16"
    D = int(rng.choice([64, 128]))
    block = int(rng.choice([128, 128, 64, 32]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Nq, Nk = int(rng.integers(1, 900)), int(rng.integers(1, 2500))
    n_forced = int(rng.integers(0, Nk + 1)) if rng.random() < 0.7 else 0
    density = float(rng.choice(DENSITIES))
    return rng, dtype, D, block, B, H, Nq, Nk, n_forced, density


@pytest.mark.parametrize("seed", range(40))
def test_random_shape(seed):
    rng, dtype, D, block, B, H, Nq, Nk, n_forced, density = _case(seed)
    log(f"random {seed}: {dtype} D={D} block={block} B={B} H={H} Nq={Nq} Nk={Nk} "
        f"forced={n_forced} density={density}")
    q = rng.standard_normal((B, H, Nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    k += np.repeat(rng.standard_normal((B, H, -(-Nk // block), D), dtype=np.float32), block, axis=2)[:, :, :Nk]
    if dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    q_t, k_t, v_t = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    res = sp.sparse_attention(q_t, k_t, v_t, n_forced, density, block=block, return_all=True)
    g_cnt, g_idx = res["kv_count"].cpu().numpy(), res["kv_index"].cpu().numpy()
    # the screened route (one call from Q and K) selects exactly the same blocks
    F_gpu = sp.forced_blocks(n_forced, block)
    c_s, i_s, qb_s, kb_s = sp.select_blocks_from_qk(q_t, k_t, F_gpu, density, block=block)
    assert np.array_equal(c_s.cpu().numpy(), g_cnt), f"seed {seed}: screened counts"
    assert np.array_equal(i_s.cpu().numpy(), g_idx), f"seed {seed}: screened selection"
    assert np.array_equal(qb_s.cpu().numpy(), res["qbar"].cpu().numpy())
    assert np.array_equal(kb_s.cpu().numpy(), res["kbar"].cpu().numpy())
    qd, kd, vd = (oracle.decode(a, dtype) for a in (q, k, v))
    S = oracle.block_scores(oracle.block_means(qd, block), oracle.block_means(kd, block))
    F = oracle.forced_blocks(n_forced, block)
    swaps = check_selection(S, F, density, g_cnt, g_idx)
    o_ref, lse_ref = oracle.sparse_attention(qd, kd, vd, g_cnt, g_idx, block)
    compare_outputs(to_f64(res["o"]), o_ref, dtype, what=f"seed {seed}")
    compare_lse(to_f64(res["lse"]), lse_ref, 1e-4 if dtype == "fp32" else 2e-3, what=f"seed {seed}")
    log(f"  rows {g_cnt.size}, near-tie swaps {swaps}")


def test_zero_budget_writes_padding():
    """No forced block and density 0: nothing is kept, the one index column
    the binding allocates holds -1, and attention gives O = 0, LSE = -inf."""
    rng = np.random.default_rng(7)
    q = bf16_bits_from_f32(rng.standard_normal((1, 2, 200, 64), dtype=np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((1, 2, 300, 64), dtype=np.float32))
    res = sp.sparse_attention(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(k, "bf16"), 0, 0.0,
                              return_all=True)
    assert np.all(res["kv_count"].cpu().numpy() == 0)
    assert np.all(res["kv_index"].cpu().numpy() == -1)
    assert np.all(to_f64(res["o"]) == 0.0)
    assert np.all(np.isneginf(to_f64(res["lse"])))


@pytest.mark.parametrize("seed", range(12))
def test_random_transfer_and_bound(seed):
    """Random geometries for the score transfer (bit-exact) and random shapes
    and budgets for the token-wise bound (within 1e-4)."""
    rng = np.random.default_rng(5000 + seed)
    block = int(rng.choice([32, 64, 128]))
    t = int(rng.integers(0, 700))
    src = (t, int(rng.integers(0 if rng.random() < 0.2 else 1, 3000)), int(rng.integers(1, 3000)))
    dst = (t, int(rng.integers(0, 3000)) if src[1] > 0 else 0, int(rng.integers(1, 3000)))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    S = rng.standard_normal((B, H, -(-src[2] // block), -(-sum(src) // block))).astype(np.float32)
    g = sp.transfer_scores(to_dev(S, "fp32"), src, dst, block=block).cpu().numpy()
    assert np.array_equal(g, oracle.transfer_scores(S, src, dst, block)), (src, dst, block)

    D = int(rng.choice([64, 128]))
    Nq, Nk = int(rng.integers(1, 600)), int(rng.integers(1, 2000))
    q = bf16_bits_from_f32(rng.standard_normal((1, H, Nq, D), dtype=np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((1, H, Nk, D), dtype=np.float32) * 1.5)
    nkb = -(-Nk // block)
    F, kb = int(rng.integers(0, nkb + 1)), int(rng.integers(0, nkb + 1))
    log(f"random transfer/bound {seed}: block={block} src={src} dst={dst}; D={D} Nq={Nq} Nk={Nk} F={F} k={kb}")
    b = to_f64(sp.token_topk_bound(to_dev(q, "bf16"), to_dev(k, "bf16"), F, kb, block=block))
    qd, kd = oracle.decode(q, "bf16"), oracle.decode(k, "bf16")
    rows = [(0, h, i) for h in range(H) for i in range(-(-Nq // block))]
    ref = oracle.token_topk_bound_rows(qd, kd, F, kb, rows, block=block)
    for (bb, h, i), m in ref.items():
        assert np.abs(b[bb, h, i * block:i * block + m.size] - m).max() <= 1e-4, (seed, h, i)
