"""fp64 CPU oracle of SparSTAR's selected-block attention -- TEST INFRASTRUCTURE.

This module is the reference the HIP library is checked against.  It is only
imported by tests, the smoke check and the benchmark's CPU baseline; it shares
no code with the GPU path and must never be called from the product path.

Sources (the pages this follows):
  [R]  "Pith review of SparSTAR: Sparse Attention for SpaceTime AutoRegressive
       Video Synthesis" (pith.science/paper/2608.10519), sections
       "What carries the argument" (means over blocks of 128 consecutive
       tokens, S_ij = tau * qbar_i^T kbar_j with tau = D^-1/2 -- Eq. 2 --,
       clip-aware retention, joint ranking, forward-only execution),
       "Core claim" (fresh block-wise Top-K per scale and head),
       "Assumptions & free parameters" (density schedule, b = 128, the SSA
       visible context text + preceding clip's final scale + current scale
       -- Eq. 1).
  [A]  "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video
       Synthesis" (mlsanity.com/paper/2608.10519), "Abstract (arXiv)":
       for each scale and head, rank key blocks by scores computed from that
       scale's own Q and K, keep the conditioning context that must stay
       visible, and compute attention over the chosen blocks only.

Readings where the pages are silent (each also listed in the design notes):
  * blocks tile the whole key sequence [text | reference | current] from token
    0; the last block of Q or K may be partial and its mean divides by its
    valid token count (the average-logit identity of [R] requires this);
  * forced context is a token prefix; a block holding any forced token is
    forced;
  * the budget is k = ceil(density * E) over the E eligible (non-forced)
    blocks, computed as one rounded fp64 product followed by ceil;
  * ties in S go to the lower block index; NaN ranks below every number;
  * attention uses scale D^-1/2, no causal mask, only keys past Nk masked;
  * the kept index list is ascending; a row with nothing kept yields O = 0
    and LSE = -inf;
  * mask reuse (the ablation baseline): blocks map between scales by the
    relative position of their centre within their segment, and the reused
    scores are ranked under the target scale's forced set and budget.

Everything is float64.  bf16 inputs are decoded exactly from their bits.
"""
import math
from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------------------
# Input decoding
# ---------------------------------------------------------------------------
def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of the stored inputs ("fp32" arrays or bf16 bits)."""
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Step 1 -- block aggregation ([R] "What carries the argument")
# ---------------------------------------------------------------------------
def block_means(x: np.ndarray, block: int = 128) -> np.ndarray:
    """x [..., N, D] -> [..., ceil(N/block), D]: mean over each block's valid tokens."""
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[-2]
    nb = -(-N // block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]), dtype=np.float64)
    for i in range(nb):
        lo, hi = i * block, min((i + 1) * block, N)
        out[..., i, :] = x[..., lo:hi, :].sum(axis=-2) / (hi - lo)
    return out


# ---------------------------------------------------------------------------
# Step 2 -- aggregated block score, Eq. 2 ([R] "What carries the argument")
# ---------------------------------------------------------------------------
def block_scores(qbar: np.ndarray, kbar: np.ndarray, tau=None) -> np.ndarray:
    """S[..., i, j] = tau * qbar_i . kbar_j, tau = D^-1/2 unless given."""
    qbar = np.asarray(qbar, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    D = qbar.shape[-1]
    if tau is None:
        tau = 1.0 / math.sqrt(D)
    lead = np.broadcast_shapes(qbar.shape[:-2], kbar.shape[:-2])
    nqb, nkb = qbar.shape[-2], kbar.shape[-2]
    S = np.empty(lead + (nqb, nkb), dtype=np.float64)
    # Elementwise products summed along D, the same reduction for every
    # (i, j): equal blocks give bit-equal scores (a BLAS product may not).
    step = max(1, (1 << 22) // max(1, nkb * D))
    for i0 in range(0, nqb, step):
        i1 = min(nqb, i0 + step)
        prod = qbar[..., i0:i1, None, :] * kbar[..., None, :, :]
        S[..., i0:i1, :] = tau * prod.sum(axis=-1)
    return S


# ---------------------------------------------------------------------------
# Step 3 -- clip-aware retention and joint Top-K ([R] "What carries the
# argument", "Core claim"; density schedule in "Assumptions & free parameters")
# ---------------------------------------------------------------------------
def forced_blocks(n_forced_tokens: int, block: int = 128) -> int:
    """Number of leading key blocks holding forced (text / Clip-1 reference) tokens."""
    return -(-int(n_forced_tokens) // block)


def budget(n_eligible: int, density: float) -> int:
    """k = ceil(density * E): one fp64 product, then ceil."""
    return int(math.ceil(float(density) * float(n_eligible)))


def kept_blocks(nkb: int, n_forced: int, density: float) -> int:
    return n_forced + budget(nkb - n_forced, density)


def select_row(s_row: np.ndarray, n_forced: int, density: float) -> np.ndarray:
    """One (batch, head, query-block) row: ascending array of kept key blocks.

    Forced blocks [0, n_forced) are always kept.  The eligible blocks (the
    reference and current blocks together) are ranked by descending score; a
    stable sort keeps lower indices first among equal scores, and NaN, which
    compares as unordered, is sorted last.
    """
    nkb = s_row.shape[0]
    eligible = np.arange(n_forced, nkb)
    k = budget(eligible.size, density)
    order = np.argsort(-s_row[n_forced:], kind="stable")   # NaN sorts last
    top = eligible[order[:k]]
    return np.sort(np.concatenate([np.arange(n_forced), top]))


def select_blocks(S: np.ndarray, n_forced: int, density: float, max_kept=None):
    """S [..., nqb, nkb] -> (kv_count [..., nqb] int32, kv_index [..., nqb, max_kept] int32).

    Rows are ascending, padded with -1.
    """
    lead = S.shape[:-1]
    nkb = S.shape[-1]
    kept = kept_blocks(nkb, n_forced, density)
    if max_kept is None:
        max_kept = kept
    flat = S.reshape(-1, nkb)
    count = np.empty(flat.shape[0], dtype=np.int32)
    index = np.full((flat.shape[0], max_kept), -1, dtype=np.int32)
    for r in range(flat.shape[0]):
        sel = select_row(flat[r], n_forced, density)
        count[r] = sel.size
        index[r, :sel.size] = sel
    return count.reshape(lead), index.reshape(lead + (max_kept,))


# ---------------------------------------------------------------------------
# Step 4 -- forward attention over the selected blocks only
# ([R] "What carries the argument": forward-only execution of the chosen blocks)
# ---------------------------------------------------------------------------
def _attend_block(q_blk, k, v, blocks, block, scale):
    """q_blk [n, D]; k, v [Nk, D]; blocks: kept key blocks.  Returns (O [n,D], LSE [n])."""
    Nk = k.shape[0]
    n, D = q_blk.shape
    if len(blocks) == 0:
        return np.zeros((n, v.shape[1])), np.full(n, -np.inf)
    keys = np.concatenate([np.arange(j * block, min((j + 1) * block, Nk)) for j in blocks])
    logits = scale * (q_blk @ k[keys].T)                 # [n, |keys|]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e / z) @ v[keys]
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def sparse_attention_rows(q, k, v, kv_count, kv_index, rows, block=128, scale=None):
    """Attention for selected query blocks only.

    q [B,H,Nq,D], k/v [B,H,Nk,D] float64; rows: iterable of (b, h, i).
    Returns {(b,h,i): (O [n,D], LSE [n])}.
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Nq = q.shape[2]
    out = {}
    for (b, h, i) in rows:
        c = int(kv_count[b, h, i])
        blocks = [int(j) for j in kv_index[b, h, i, :c]]
        qb = q[b, h, i * block:min((i + 1) * block, Nq)]
        out[(b, h, i)] = _attend_block(qb, k[b, h], v[b, h], blocks, block, scale)
    return out


def sparse_attention(q, k, v, kv_count, kv_index, block=128, scale=None):
    """Full O [B,H,Nq,D] and LSE [B,H,Nq] for every query block."""
    B, H, Nq, D = q.shape
    nqb = -(-Nq // block)
    o = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nqb)]
    res = sparse_attention_rows(q, k, v, kv_count, kv_index, rows, block, scale)
    for (b, h, i), (ob, lb) in res.items():
        o[b, h, i * block:i * block + ob.shape[0]] = ob
        lse[b, h, i * block:i * block + ob.shape[0]] = lb
    return o, lse


# ---------------------------------------------------------------------------
# Diagnostic -- retained attention mass and the token-wise Top-K bound
# ([R] "Core claim": block-wise Top-K recomputed per scale is compared with a
# token-wise upper bound by the attention mass it retains; [R] "Editorial
# extensions": an exact per-token Top-K selection at equal density as the
# reference point)
# ---------------------------------------------------------------------------
def _dense_probs(q_blk, k, scale):
    """Dense softmax rows p[t, s] of one query block over all Nk keys."""
    logits = scale * (q_blk @ k.T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True)


def retained_mass_rows(q, k, kv_count, kv_index, rows, block=128, scale=None):
    """Retained attention mass of the kept blocks, per query token.

    For query t of block i: the sum, over the valid keys of the kept blocks,
    of t's dense softmax probabilities (softmax over all Nk keys).  1 when
    every block is kept.  Returns {(b,h,i): mass [n]}.
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Nq, Nk = q.shape[2], k.shape[2]
    out = {}
    for (b, h, i) in rows:
        qb = q[b, h, i * block:min((i + 1) * block, Nq)]
        p = _dense_probs(qb, k[b, h], scale)
        c = int(kv_count[b, h, i])
        keep = np.zeros(Nk, dtype=bool)
        for j in kv_index[b, h, i, :c]:
            if 0 <= j and j * block < Nk:
                keep[j * block:min((j + 1) * block, Nk)] = True
        out[(b, h, i)] = p[:, keep].sum(axis=1)
    return out


def token_topk_bound_rows(q, k, n_forced_blocks, k_blocks, rows, block=128, scale=None):
    """Token-wise Top-K upper bound at the same budget, per query token.

    The block policy keeps the forced prefix blocks and k_blocks eligible
    blocks, i.e. at most k_blocks * block eligible tokens.  The token-wise
    policy keeps the same forced tokens and, per query token, the
    k_blocks * block eligible keys of largest dense probability; its retained
    mass bounds the block policy's from above.  Returns {(b,h,i): bound [n]}.
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Nq, Nk = q.shape[2], k.shape[2]
    f_tok = min(n_forced_blocks * block, Nk)
    m_tok = min(k_blocks * block, Nk - f_tok)
    out = {}
    for (b, h, i) in rows:
        qb = q[b, h, i * block:min((i + 1) * block, Nq)]
        p = _dense_probs(qb, k[b, h], scale)
        forced = p[:, :f_tok].sum(axis=1)
        elig = np.sort(p[:, f_tok:], axis=1)[:, ::-1]
        out[(b, h, i)] = forced + elig[:, :m_tok].sum(axis=1)
    return out


# ---------------------------------------------------------------------------
# Mask reuse -- the ablation baseline the method is compared against
# ([R] "Extended reading notes", "Core claim": a block selection carried over
# from another scale, or across a clip boundary, keeps less attention mass
# than a fresh one; [A] "Abstract (arXiv)": the paper's analyses compare a
# selection computed anew per scale with one carried over).
#
# The pages do not say how block indices map between scales.  Reading: a
# scale's geometry is (n_text, n_ref, n_cur); queries are the current scale
# and keys the concatenation [text | ref | cur] (Eq. 1 order).  A block is
# represented by the centre of its valid tokens (token t covers [t, t + 1));
# the segment holding that centre is mapped by relative position onto the
# same segment of the other scale, and the token found there names the block.
# The transferred selection ranks the target scale's eligible blocks by the
# scores of the blocks they map to, under the target scale's own forced set
# and budget (so both selections spend the same number of blocks), with the
# usual tie rule.
# ---------------------------------------------------------------------------
def _centre(j, n_tokens, block):
    """Centre of the valid tokens of block j of an n_tokens sequence (exact)."""
    first = j * block
    last = min((j + 1) * block, n_tokens) - 1
    return Fraction(first + last + 1, 2)


def transfer_query_map(src_n_cur, dst_n_cur, block=128):
    """For each target query block, the source query block it reuses."""
    if src_n_cur < 1 or dst_n_cur < 1:
        raise ValueError("both scales need at least one query token")
    nqb_dst = -(-dst_n_cur // block)
    out = np.empty(nqb_dst, dtype=np.int64)
    for i in range(nqb_dst):
        rel = _centre(i, dst_n_cur, block) / dst_n_cur
        out[i] = math.floor(rel * src_n_cur) // block
    return out


def transfer_key_map(src_geom, dst_geom, block=128):
    """For each target key block, the source key block it reuses.

    src_geom, dst_geom: (n_text, n_ref, n_cur) of the two scales."""
    src = [int(x) for x in src_geom]
    dst = [int(x) for x in dst_geom]
    if min(src + dst) < 0:
        raise ValueError("segment lengths must be non-negative")
    n_dst = sum(dst)
    nkb_dst = -(-n_dst // block)
    out = np.empty(nkb_dst, dtype=np.int64)
    for j in range(nkb_dst):
        c = _centre(j, n_dst, block)
        start_dst = start_src = 0
        for seg in range(3):
            if start_dst <= c < start_dst + dst[seg]:
                if src[seg] == 0:
                    raise ValueError("a target segment has no counterpart in the source scale")
                rel = (c - start_dst) / dst[seg]
                out[j] = (start_src + math.floor(rel * src[seg])) // block
                break
            start_dst += dst[seg]
            start_src += src[seg]
    return out


def transfer_scores(S_src, src_geom, dst_geom, block=128):
    """S_src [..., nqb_src, nkb_src] -> the scores each target block pair reuses."""
    qmap = transfer_query_map(int(src_geom[2]), int(dst_geom[2]), block)
    kmap = transfer_key_map(src_geom, dst_geom, block)
    S_src = np.asarray(S_src)
    return S_src[..., qmap[:, None], kmap[None, :]]


def transferred_selection(S_src, src_geom, dst_geom, n_forced, density, block=128,
                          max_kept=None):
    """The target scale's selection when the source scale's scores are reused."""
    return select_blocks(transfer_scores(S_src, src_geom, dst_geom, block), n_forced,
                         density, max_kept)


# ---------------------------------------------------------------------------
# Whole path and counting helpers
# ---------------------------------------------------------------------------
def run_pipeline(q, k, v, n_forced_tokens, density, block=128, attention=True):
    """means -> scores -> selection (-> attention) for float64 q, k, v."""
    qbar = block_means(q, block)
    kbar = block_means(k, block)
    S = block_scores(qbar, kbar)
    F = forced_blocks(n_forced_tokens, block)
    count, index = select_blocks(S, F, density)
    res = {"qbar": qbar, "kbar": kbar, "S": S, "n_forced": F,
           "kv_count": count, "kv_index": index}
    if attention:
        res["o"], res["lse"] = sparse_attention(q, k, v, count, index, block)
    return res


def selected_flops(kv_count, kv_index, Nq, Nk, D, block=128):
    """4 * D * sum over rows of (valid queries) x (valid keys in kept blocks)."""
    counts = np.asarray(kv_count).reshape(-1)
    idx = np.asarray(kv_index).reshape(counts.size, -1)
    nqb = -(-Nq // block)
    total = 0
    for r in range(counts.size):
        i = r % nqb
        nq = min((i + 1) * block, Nq) - i * block
        blocks = idx[r, :counts[r]]
        nk = int(np.minimum((blocks + 1) * block, Nk).sum() - (blocks * block).sum())
        total += 4 * D * nq * nk
    return total
