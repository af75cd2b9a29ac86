"""Seeded inputs with concentrated attention: the logits of successive kept
key blocks rise in steps of many log2 units, as in the peaked attention of
real video activations (SparSTAR review, "Core claim": block-wise Top-K keeps
almost all of the attention mass because it is concentrated in few blocks).

This module only lays out random numbers (no means, scores, selection or
attention).  The layout:

* every key block j gets a logit level lev[j] (log2 units), realised as
  k_s[0] = lev[j] * ln 2 / (scale * alpha) for the keys of block j, with
  q_t[0] = alpha * (1 + 0.02 n_t) for every query; the remaining coordinates
  are N(0, 1) for keys and N(0, sigma^2) for queries, which spreads the
  logits of one block by about sigma nats;
* two families of index lists, given in processing order (not sorted):
  - "stairs" (query blocks 0 and 1, sigma 0.7): two low blocks (level 0),
    eight plateau blocks (level 8), then one block at each of the levels
    17, 35 and 53, and last the partial last key block, whose first tiles
    sit at level 56 and whose last, partial tile sits at level 78;
  - "comparable" (query block 2, sigma 0.15): two low blocks, eight blocks
    of a second plateau and two "near" blocks, the levels chosen from the
    tile size so that a plateau tile sums to about 2^14.3 and a near tile to
    about 2^18 against the first tile's maximum: the near tiles move the
    reference once, and the plateau's rescaled mass stays a large share of
    the total;
  the blocks of each class are drawn at random per row.

V is N(0, 1).  bf16 cases round every value to bfloat16 (nearest-even).
"""
import math

import numpy as np

from .generate import bf16_bits_from_f32

ALPHA = 8.0
SIGMA_STAIRS, SIGMA_COMPARABLE = 0.7, 0.15
LAST_LEVEL, LAST_TILE_LEVEL = 56.0, 78.0


def last_tile_keys(block: int) -> int:
    """Keys per LDS tile of the bf16 attention kernel: 64 for 128-token
    blocks, 32 below (the partial last tile is where the last level rises)."""
    return 64 if block >= 128 else 32


def classes(block: int):
    """(name, level, blocks in the class, blocks a row of its family takes, family)."""
    lt = math.log2(last_tile_keys(block))
    return (("low", 0.0, 4, 2, "both"), ("plateau", 8.0, 12, 8, "stairs"),
            ("cross", 17.0, 2, 1, "stairs"), ("stair1", 35.0, 2, 1, "stairs"),
            ("stair2", 53.0, 2, 1, "stairs"),
            ("plateau_b", 14.3 - lt + 0.5, 12, 8, "comparable"),
            ("near", 18.0 - lt + 0.5, 2, 2, "comparable"))


def concentrated_case(dtype: str, D: int, block: int, seed: int, B: int = 1, H: int = 2):
    """Returns a dict with q, k, v (bf16 bits or float32 arrays), kv_count,
    kv_index (int32, processing order, -1 padded), the per-key levels, the
    family of each query block and the sizes."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    tile = last_tile_keys(block)
    cls = classes(block)
    # the last key block is partial and its last tile is partial too
    last_valid = tile + tile // 4 if block > tile else (3 * block) // 4 - 4
    nkb = sum(c[2] for c in cls) + 1
    Nk = (nkb - 1) * block + last_valid
    Nq = 2 * block + block // 2 - 12            # three query blocks, the last partial
    nqb = -(-Nq // block)
    family = ["stairs", "stairs", "comparable"]
    f32 = np.float32

    # key levels, block by block (classes in a shuffled block order)
    order = rng.permutation(nkb - 1)
    level_of_block = np.empty(nkb)
    members = {}
    pos = 0
    for name, lev, n, _, _ in cls:
        blocks = np.sort(order[pos:pos + n])
        members[name] = blocks
        level_of_block[blocks] = lev
        pos += n
    level_of_block[nkb - 1] = LAST_LEVEL
    key_level = np.repeat(level_of_block, block)[:Nk].copy()
    part0 = (nkb - 1) * block + (last_valid // tile) * tile   # first key of the partial tile
    key_level[part0:] = LAST_TILE_LEVEL

    q = rng.standard_normal((B, H, Nq, D), dtype=f32)
    k = rng.standard_normal((B, H, Nk, D), dtype=f32)
    v = rng.standard_normal((B, H, Nk, D), dtype=f32)
    sigma = np.repeat(np.array([SIGMA_STAIRS if f == "stairs" else SIGMA_COMPARABLE
                                for f in family], dtype=f32), block)[:Nq]
    q *= sigma[None, None, :, None]
    q[..., 0] = f32(ALPHA) * (1 + f32(0.02) * rng.standard_normal((B, H, Nq), dtype=f32))
    k[..., 0] = (key_level * math.log(2.0) / (scale * ALPHA)).astype(f32)[None, None, :]

    takes = {f: sum(c[3] for c in cls if c[4] in (f, "both")) for f in ("stairs", "comparable")}
    max_kept = takes["stairs"] + 1
    kv_index = np.full((B, H, nqb, max_kept), -1, dtype=np.int32)
    kv_count = np.zeros((B, H, nqb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                row = []
                for name, _, _, take, fam in cls:
                    if fam in (family[i], "both"):
                        row += list(rng.choice(members[name], size=take, replace=False))
                if family[i] == "stairs":
                    row.append(nkb - 1)
                kv_index[b, h, i, :len(row)] = row
                kv_count[b, h, i] = len(row)
    if dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return {"q": q, "k": k, "v": v, "kv_count": kv_count, "kv_index": kv_index,
            "key_level": key_level, "family": family, "classes": cls, "B": B, "H": H,
            "Nq": Nq, "Nk": Nk, "D": D, "block": block, "dtype": dtype, "scale": scale}
