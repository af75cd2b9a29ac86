"""Concentrated attention: index lists whose logits rise by many log2 units
from tile to tile, so that the bf16 kernel's softmax reference max has to
move after the first tile (several times per row, the last time on the
partial last tile), and lists where a long plateau of tiles stays under the
move threshold before a tile crosses it, so that the rescaled old mass is a
large share of the total (a wrong rescale factor shows in the output).
Outputs and LSE are compared with the oracle, query by query.

The bf16 kernel keeps a per-query reference max from the first tile and only
moves it when a tile's bf16 weights, summed over the tile, would exceed 2^16;
the decision is taken for a whole wave of 32 queries.  `replay_moves`
re-enacts that rule in float64 on the CPU, so each case proves that its
inputs take the move path the required number of times; it refuses inputs
that fall within a factor 2 of the threshold, where rounding could decide
the kernel's path differently from the replay.
"""
import numpy as np
import pytest

import oracle
from tests.parity_util import compare_lse, compare_outputs, log, to_dev, to_f64
from workloads.concentrated import concentrated_case, last_tile_keys

ROW_SUM_LIMIT = 65536.0          # the kernel's threshold on a tile's weight sum
CASES = [("bf16", D, blk) for D in (64, 128) for blk in (128, 64, 32)] + \
        [("fp32", D, blk) for D in (64, 128) for blk in (128, 32)]


def replay_moves(c):
    """Per wave (b, h, query block, wave): the list of tile numbers at which
    the bf16 kernel moves its reference max after the first tile, and the
    number of tiles processed.  Raises if a tile's largest row sum over the
    wave lies within a factor 2 of the threshold."""
    qd = oracle.decode(c["q"], c["dtype"])
    kd = oracle.decode(c["k"], c["dtype"])
    block, Nq, Nk = c["block"], c["Nq"], c["Nk"]
    tile = last_tile_keys(block)
    sl2 = c["scale"] / np.log(2.0)
    nkb = -(-Nk // block)
    out = {}
    for b in range(c["B"]):
        for h in range(c["H"]):
            for i in range(c["kv_count"].shape[2]):
                lst = c["kv_index"][b, h, i, :c["kv_count"][b, h, i]]
                tiles = []
                for j in lst:
                    if not 0 <= j < nkb:
                        continue
                    for p in range(block // tile):
                        k0 = j * block + p * tile
                        if k0 < Nk:
                            tiles.append((k0, min(k0 + tile, Nk)))
                for w in range(block // 32):
                    t0 = i * block + 32 * w
                    t1 = min(t0 + 32, Nq)
                    if t0 >= t1:
                        continue
                    q = qd[b, h, t0:t1]
                    m_ref = None
                    moves = []
                    for n, (k0, k1) in enumerate(tiles):
                        s = sl2 * (q @ kd[b, h, k0:k1].T)          # [queries, keys], log2 units
                        tmax = s.max(axis=1)
                        if m_ref is None:
                            m_ref = tmax
                            continue
                        r = np.exp2(s - m_ref[:, None]).sum(axis=1).max()
                        if ROW_SUM_LIMIT / 2 <= r <= 2 * ROW_SUM_LIMIT:
                            raise AssertionError(f"tile {n} of wave {(b, h, i, w)} is within a "
                                                 f"factor 2 of the threshold (row sum {r:.3g})")
                        if r > ROW_SUM_LIMIT:
                            moves.append(n)
                            m_ref = np.maximum(m_ref, tmax)
                    out[(b, h, i, w)] = (moves, len(tiles))
    return out


def plateau_share(c):
    """Per query of the "comparable" rows: the softmax mass of the second
    plateau's keys (float64, from the decoded inputs)."""
    qd = oracle.decode(c["q"], c["dtype"])
    kd = oracle.decode(c["k"], c["dtype"])
    block, Nq, Nk = c["block"], c["Nq"], c["Nk"]
    lev_b = [lev for name, lev, *_ in c["classes"] if name == "plateau_b"][0]
    shares = []
    for b in range(c["B"]):
        for h in range(c["H"]):
            for i, fam in enumerate(c["family"]):
                if fam != "comparable" or i * block >= Nq:
                    continue
                lst = c["kv_index"][b, h, i, :c["kv_count"][b, h, i]]
                keys = np.concatenate([np.arange(j * block, min((j + 1) * block, Nk)) for j in lst])
                s = c["scale"] * (qd[b, h, i * block:min((i + 1) * block, Nq)] @ kd[b, h, keys].T)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                shares.append(p[:, c["key_level"][keys] == lev_b].sum(axis=1))
    return np.concatenate(shares)


def check_crossings(c):
    """The inputs take the move path as designed: "stairs" waves at least
    four times (never on the plateau, the last time on the partial last
    tile), "comparable" waves at least once, and there the plateau keeps at
    least a fifth of every query's mass."""
    moves = replay_moves(c)
    tpb = c["block"] // last_tile_keys(c["block"])
    for key, (mv, n_tiles) in moves.items():
        if c["family"][key[2]] == "stairs":
            assert len(mv) >= 4, (key, mv)
            assert min(mv) >= 10 * tpb, (key, mv)
            assert mv[-1] == n_tiles - 1, (key, mv, n_tiles)
        else:
            assert len(mv) >= 1 and min(mv) >= 10 * tpb, (key, mv)
    share = plateau_share(c)
    assert share.min() >= 0.2, float(share.min())
    return moves, share


@pytest.mark.parametrize("dtype,D,block", CASES)
def test_inputs_cross_the_threshold(dtype, D, block):
    """CPU: the replayed kernel rule moves the reference max as designed
    (checked for the fp32 inputs too, which share the layout)."""
    check_crossings(concentrated_case(dtype, D, block, seed=D + block))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block", CASES)
def test_concentrated_attention(dtype, D, block):
    import torch
    import block_sparse_attention_head_amd as sp
    c = concentrated_case(dtype, D, block, seed=D + block)
    moves, share = check_crossings(c)
    n_moves = sum(len(m) for m, _ in moves.values())
    log(f"concentrated {dtype} D={D} block={block}: Nq={c['Nq']} Nk={c['Nk']}, "
        f"{len(moves)} waves, {n_moves} reference-max moves after the first tile (replayed), "
        f"plateau share of the comparable rows >= {float(share.min()):.2f}")
    cnt_t = torch.from_numpy(c["kv_count"]).cuda()
    idx_t = torch.from_numpy(c["kv_index"]).cuda()
    o, lse = sp.block_sparse_attn_fwd(to_dev(c["q"], dtype), to_dev(c["k"], dtype),
                                      to_dev(c["v"], dtype), cnt_t, idx_t, block=block)
    qd, kd, vd = (oracle.decode(c[n], dtype) for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.sparse_attention(qd, kd, vd, c["kv_count"], c["kv_index"], block)
    mx, rel = compare_outputs(to_f64(o), o_ref, dtype, f"{dtype} D={D} block={block}")
    compare_lse(to_f64(lse), lse_ref, 1e-4 if dtype == "fp32" else 2e-3, "lse")
    log(f"  max|dO|={mx:.3g} relL2={rel} max|dLSE|={float(np.abs(to_f64(lse) - lse_ref).max()):.3g}")


def _lazy_softmax(c, mutation=None):
    """float64 model of the bf16 kernel's softmax bookkeeping (reference max
    from the first tile, moved by the wave-wide 2^16 rule), with an optional
    planted mistake in the rescale; returns O and LSE like the kernel."""
    qd, kd, vd = (oracle.decode(c[n], c["dtype"]) for n in ("q", "k", "v"))
    block, Nq, Nk = c["block"], c["Nq"], c["Nk"]
    tile = last_tile_keys(block)
    sl2 = c["scale"] / np.log(2.0)
    o = np.zeros(qd.shape)
    lse = np.zeros(qd.shape[:3])
    for b in range(c["B"]):
        for h in range(c["H"]):
            for i in range(c["kv_count"].shape[2]):
                lst = c["kv_index"][b, h, i, :c["kv_count"][b, h, i]]
                tiles = [(j * block + p * tile, min(j * block + (p + 1) * tile, Nk))
                         for j in lst for p in range(block // tile) if j * block + p * tile < Nk]
                for t0 in range(i * block, min((i + 1) * block, Nq), 32):
                    t1 = min(t0 + 32, Nq)
                    q = qd[b, h, t0:t1]
                    m_ref = np.full(t1 - t0, -np.inf)
                    l_run = np.zeros(t1 - t0)
                    acc = np.zeros((t1 - t0, vd.shape[-1]))
                    for (k0, k1) in tiles:
                        s = sl2 * (q @ kd[b, h, k0:k1].T)
                        first = np.isneginf(m_ref[0])
                        p = None if first else np.exp2(s - m_ref[:, None])
                        if first or p.sum(axis=1).max() > ROW_SUM_LIMIT:
                            m_new = np.maximum(m_ref, s.max(axis=1))
                            alpha = np.exp2(m_ref - m_new)
                            if mutation == "natural_base":
                                alpha = np.exp(m_ref - m_new)
                            if mutation != "l_not_rescaled":
                                l_run = l_run * alpha
                            if mutation != "o_not_rescaled":
                                acc = acc * alpha[:, None]
                            m_ref = m_new
                            p = np.exp2(s - m_ref[:, None])
                        l_run += p.sum(axis=1)
                        acc += p @ vd[b, h, k0:k1]
                    o[b, h, t0:t1] = acc / l_run[:, None]
                    lse[b, h, t0:t1] = (m_ref + np.log2(l_run)) * np.log(2.0)
    return o, lse


@pytest.mark.parametrize("mutation", [None, "natural_base", "l_not_rescaled", "o_not_rescaled"])
def test_cases_detect_a_wrong_rescale(mutation):
    """CPU: on these inputs a float64 model of the kernel's bookkeeping
    matches the oracle within the bf16 tolerances, and each planted rescale
    mistake in the model breaks them (so the GPU test above can see it)."""
    c = concentrated_case("bf16", 128, 128, seed=256)
    o, lse = _lazy_softmax(c, mutation)
    qd, kd, vd = (oracle.decode(c[n], "bf16") for n in ("q", "k", "v"))
    o_ref, lse_ref = oracle.sparse_attention(qd, kd, vd, c["kv_count"], c["kv_index"], 128)
    if mutation is None:
        compare_outputs(o, o_ref, "bf16", "model")
        compare_lse(lse, lse_ref, 2e-3, "model")
    else:
        with pytest.raises(AssertionError):
            compare_outputs(o, o_ref, "bf16", "model")
            compare_lse(lse, lse_ref, 2e-3, "model")
