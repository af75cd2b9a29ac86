"""GPU parity of the mask-reuse baseline: score transfer between scales (and
across a clip boundary) and the selection made from transferred scores,
against the oracle.  Every call goes through the C ABI (ctypes binding)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_head_amd as sp
import oracle
from tests.parity_util import check_selection, log, to_dev, to_f64
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.gpu


def _scores(B, H, geom, block, seed):
    nqb = -(-geom[2] // block)
    nkb = -(-sum(geom) // block)
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, H, nqb, nkb)).astype(np.float32)


GEOMS = [
    # (src, dst): upsampling, downsampling, identity (a clip boundary at one
    # scale), partial blocks, a block straddling segments, empty reference
    ((512, 1000, 1300), (512, 2300, 2900)),
    ((512, 2300, 2900), (512, 1000, 1300)),
    ((512, 3600, 3000), (512, 3600, 3000)),
    ((100, 333, 77), (100, 1001, 130)),
    ((0, 0, 500), (0, 0, 1700)),
    ((300, 200, 200), (300, 0, 900)),
    ((1, 1, 1), (1, 5000, 300)),
]


@pytest.mark.parametrize("block", [128, 64, 32])
@pytest.mark.parametrize("src,dst", GEOMS)
def test_transfer_scores_bit_exact(src, dst, block):
    log(f"transfer src={src} dst={dst} block={block}")
    S = _scores(2, 3, src, block, seed=sum(src) + block)
    g = sp.transfer_scores(torch.from_numpy(S).cuda(), src, dst, block=block).cpu().numpy()
    ref = oracle.transfer_scores(S, src, dst, block)
    assert g.shape == ref.shape
    assert np.array_equal(g, ref)


@pytest.mark.parametrize("src,dst", [
    ((512, 18000, 18000), (512, 72000, 72000)),     # 18k scale reused at 72k
    ((512, 72000, 72000), (512, 18000, 18000)),
    ((512, 72000, 72000), (512, 72000, 72000)),     # across a clip boundary, 72k
    ((512, 32000, 32000), (512, 72000, 72000)),
])
def test_transfer_scores_full_size(src, dst):
    log(f"transfer full size src={src} dst={dst}")
    S = _scores(1, 16, src, 128, seed=7)
    g = sp.transfer_scores(torch.from_numpy(S).cuda(), src, dst).cpu().numpy()
    ref = oracle.transfer_scores(S, src, dst)
    assert np.array_equal(g, ref)


@pytest.mark.parametrize("src,dst,F,density", [
    ((512, 1000, 1300), (512, 2300, 2900), 4, 0.1875),
    ((512, 18000, 18000), (512, 72000, 72000), 4, 0.09375),
    ((512, 32000, 32000), (512, 72000, 72000), 4, 0.09375),
    ((512, 3600, 3000), (512, 3600, 3000), 33, 0.25),
    ((0, 0, 500), (0, 0, 1700), 0, 0.0),
    ((300, 200, 200), (300, 0, 900), 3, 1.0),
])
def test_transferred_selection_bit_exact(src, dst, F, density):
    """Both sides rank the same fp32 values; the transferred scores hold exact
    duplicates (one source block feeds several target blocks), so this also
    checks the tie rule (lower block index first) on many ties."""
    log(f"transferred selection src={src} dst={dst} F={F} density={density}")
    S = _scores(1, 16 if sum(dst) > 50000 else 2, src, 128, seed=len(str(src)) + F)
    mk = max(1, sp.kept_blocks(-(-sum(dst) // 128), F, density))   # -1 padding is checked too
    gc, gi = sp.transferred_selection(torch.from_numpy(S).cuda(), src, dst, F, density, max_kept=mk)
    rc, ri = oracle.transferred_selection(S.astype(np.float64), src, dst, F, density, max_kept=mk)
    assert np.array_equal(gc.cpu().numpy(), rc)
    assert np.array_equal(gi.cpu().numpy(), ri)


def test_mask_reuse_end_to_end():
    """Two small scales of one clip: the source scale's scores computed on the
    GPU from its Q and K, carried to the target scale, selected under the
    target's budget; checked against the oracle's transferred selection from
    its own fp64 scores, then the retained mass of the reused and of the fresh
    selection against the oracle on every row."""
    rng = np.random.default_rng(21)
    B, H, D, text, F_tok, density = 1, 2, 128, 256, 256, 0.1875
    src, dst = (text, 1000, 1000), (text, 2100, 2100)

    def draw(geom):
        q = rng.standard_normal((B, H, geom[2], D), dtype=np.float32)
        k = rng.standard_normal((B, H, sum(geom), D), dtype=np.float32)
        v = rng.standard_normal((B, H, sum(geom), D), dtype=np.float32)
        # per-block offsets give the ranking some structure
        for x, n in ((q, geom[2]), (k, sum(geom))):
            off = rng.standard_normal((B, H, -(-n // 128), D), dtype=np.float32) * 0.5
            x += np.repeat(off, 128, axis=2)[:, :, :n]
        return [bf16_bits_from_f32(a) for a in (q, k, v)]

    qs, ks, _ = draw(src)
    qt, kt, vt = draw(dst)
    S_src_g = sp.block_scores(sp.block_means(to_dev(qs, "bf16")), sp.block_means(to_dev(ks, "bf16")))
    F = sp.forced_blocks(F_tok)
    gc, gi = sp.transferred_selection(S_src_g, src, dst, F, density)
    qsd, ksd = oracle.decode(qs, "bf16"), oracle.decode(ks, "bf16")
    S_src_o = oracle.block_scores(oracle.block_means(qsd), oracle.block_means(ksd))
    S_t = oracle.transfer_scores(S_src_o, src, dst)
    swaps = check_selection(S_t, F, density, gc.cpu().numpy(), gi.cpu().numpy())
    log(f"  near-tie swaps: {swaps}")

    qd, kd, vd = (to_dev(a, "bf16") for a in (qt, kt, vt))
    m_reuse = to_f64(sp.selection_retained_mass(qd, kd, vd, gc, gi))
    fresh = sp.sparse_attention(qd, kd, vd, F_tok, density, return_all=True)
    m_fresh = to_f64(sp.selection_retained_mass(qd, kd, vd, fresh["kv_count"], fresh["kv_index"]))
    qo, ko = oracle.decode(qt, "bf16"), oracle.decode(kt, "bf16")
    rows = [(0, h, i) for h in range(H) for i in range(-(-dst[2] // 128))]
    ref = oracle.retained_mass_rows(qo, ko, gc.cpu().numpy(), gi.cpu().numpy(), rows)
    worst = max(float(np.abs(m_reuse[b, h, i * 128:i * 128 + m.size] - m).max())
                for (b, h, i), m in ref.items())
    log(f"  reused mass {m_reuse.mean():.4f} fresh {m_fresh.mean():.4f}; max |gpu - oracle| {worst:.3g}")
    assert worst <= 5e-3
    assert np.all(m_reuse >= 0) and np.all(m_reuse <= 1 + 1e-6)
