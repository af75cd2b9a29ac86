"""GPU parity of the token-wise Top-K upper bound (the retained-mass
diagnostic's reference point) against the oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_head_amd as sp
import oracle
from tests.parity_util import log, to_dev, to_f64
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

# logits from bf16 MFMA with float32 accumulation against float64, sums in
# float32, and an upward error below 1e-5 relative from the last bisection
# interval: 1e-4 absolute on a mass in [0, 1]
TOL = 1e-4


def _qk(B, H, Nq, Nk, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    # per-block offsets give the attention some concentration
    q += np.repeat(rng.standard_normal((B, H, -(-Nq // 128), D), dtype=np.float32) * 0.4, 128, axis=2)[:, :, :Nq]
    k += np.repeat(rng.standard_normal((B, H, -(-Nk // 128), D), dtype=np.float32) * 0.6, 128, axis=2)[:, :, :Nk]
    return bf16_bits_from_f32(q), bf16_bits_from_f32(k)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(300, 700), (129, 1000), (256, 300)])
@pytest.mark.parametrize("F,kb", [(2, 1), (0, 2), (1, 0), (0, 0), (1, 100)])
def test_token_bound_matches_oracle(D, Nq, Nk, F, kb):
    log(f"token bound D={D} Nq={Nq} Nk={Nk} F={F} k={kb}")
    q, k = _qk(1, 2, Nq, Nk, D, seed=Nq + Nk + D + F)
    g = to_f64(sp.token_topk_bound(to_dev(q, "bf16"), to_dev(k, "bf16"), F, kb))
    qd, kd = oracle.decode(q, "bf16"), oracle.decode(k, "bf16")
    rows = [(0, h, i) for h in range(2) for i in range(-(-Nq // 128))]
    ref = oracle.token_topk_bound_rows(qd, kd, F, kb, rows)
    worst = 0.0
    for (b, h, i), m in ref.items():
        got = g[b, h, i * 128:i * 128 + m.size]
        worst = max(worst, float(np.abs(got - m).max()))
    log(f"  max |bound - oracle| = {worst:.3g}")
    assert worst <= TOL


def test_token_bound_bounds_the_block_selection():
    """At the same budget the token-wise bound is at least the retained mass
    of the block selection, query by query; at a full budget both are 1."""
    Nq, Nk, D = 1000, 3000, 128
    q, k = _qk(1, 3, Nq, Nk, D, seed=5)
    rng = np.random.default_rng(6)
    v = bf16_bits_from_f32(rng.standard_normal((1, 3, Nk, D), dtype=np.float32))
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    for n_forced_tokens, density in [(256, 0.1875), (0, 0.25), (130, 1.0)]:
        res = sp.sparse_attention(qd, kd, vd, n_forced_tokens, density, return_all=True)
        F = sp.forced_blocks(n_forced_tokens)
        kept = int(res["kv_count"].reshape(-1)[0])
        mass = to_f64(sp.selection_retained_mass(qd, kd, vd, res["kv_count"], res["kv_index"]))
        bound = to_f64(sp.token_topk_bound(qd, kd, F, kept - F))
        log(f"  forced={n_forced_tokens} density={density}: mass {mass.mean():.4f} bound {bound.mean():.4f}")
        assert np.all(bound >= mass - 1e-5)
        if density == 1.0:
            assert np.all(bound == 1.0) and np.abs(mass - 1).max() <= 1e-6


def test_token_bound_sampled_rows_at_mid_scale():
    """A larger head (2 heads, 18,000 queries, 36,512 keys) on sampled query
    blocks against the oracle."""
    from workloads import make_inputs
    from workloads.configs import MID
    import dataclasses
    w = dataclasses.replace(MID, H=2, name="mid-18k-2h")
    x = make_inputs(w)
    F = sp.forced_blocks(w.n_forced_tokens)
    kb = 53
    g = to_f64(sp.token_topk_bound(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), F, kb))
    qd, kd = oracle.decode(x["q"], "bf16"), oracle.decode(x["k"], "bf16")
    rows = [(0, h, i) for h in range(2) for i in (0, 70, 140)]
    ref = oracle.token_topk_bound_rows(qd, kd, F, kb, rows)
    worst = max(float(np.abs(g[b, h, i * 128:i * 128 + m.size] - m).max()) for (b, h, i), m in ref.items())
    log(f"  mid scale: max |bound - oracle| = {worst:.3g}")
    assert worst <= TOL
