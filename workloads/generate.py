"""Deterministic input generator (numpy PCG64, seed per workload).

Recipe, in draw order (all draws float32):
  1. Q [B,H,Nq,D], K [B,H,Nk,D], V [B,H,Nk,D] ~ N(0, 1).
  2. Per-block mean offsets ~ N(0, offset_std^2)^D: for Q blocks (if
     offset_q), for K blocks, for V blocks (if offset_v), each block of
     ``block`` consecutive tokens sharing one offset vector; the last block of
     a sequence may be partial.
  3. Shifted key blocks: for each (b, h), round(shift_frac * nkb) key blocks
     chosen uniformly without replacement get shift_amount * u_bh added to
     every token, u_bh being the unit vector along the mean of all query
     tokens of that (b, h) (taken after step 2).
  4. bf16 workloads round every float32 value to bfloat16 (round to nearest,
     ties to even) and hand out the raw 16-bit patterns.

The arrays returned are what both the GPU path and the oracle consume:
float32 arrays for "fp32" workloads, uint16 bf16 bit patterns for "bf16".
"""
import numpy as np

from .configs import Workload


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite, so no NaN special case is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1).view(np.uint32)
    flat_out = out.reshape(-1)
    step = 1 << 22
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step]
        r = (u >> 16) & 1
        r += 0x7FFF
        r += u                      # finite inputs: no uint32 wrap-around
        r >>= 16
        flat_out[s:s + step] = r
    return out


def _add_block_offsets(x: np.ndarray, off: np.ndarray, block: int) -> None:
    """x[..., t, :] += off[..., t // block, :] in place."""
    B, H, N, D = x.shape
    nfull = N // block
    if nfull:
        x[:, :, :nfull * block, :].reshape(B, H, nfull, block, D)[...] += off[:, :, :nfull, None, :]
    if N % block:
        x[:, :, nfull * block:, :] += off[:, :, nfull:nfull + 1, :]


def make_inputs(w: Workload, seed=None) -> dict:
    """Draw Q, K, V for workload ``w``.  Returns a dict with the arrays and sizes."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, H, D, Nq, Nk, b = w.B, w.H, w.D, w.Nq, w.Nk, w.block
    nqb, nkb = w.nqb, w.nkb
    f32 = np.float32
    q = rng.standard_normal((B, H, Nq, D), dtype=f32)
    k = rng.standard_normal((B, H, Nk, D), dtype=f32)
    v = rng.standard_normal((B, H, Nk, D), dtype=f32)
    if w.offset_q:
        _add_block_offsets(q, rng.standard_normal((B, H, nqb, D), dtype=f32) * f32(w.offset_std), b)
    _add_block_offsets(k, rng.standard_normal((B, H, nkb, D), dtype=f32) * f32(w.offset_std), b)
    if w.offset_v:
        _add_block_offsets(v, rng.standard_normal((B, H, nkb, D), dtype=f32) * f32(w.offset_std), b)
    n_shift = int(round(w.shift_frac * nkb))
    shifted = np.zeros((B, H, n_shift), dtype=np.int64)
    if n_shift:
        qmean = q.mean(axis=2, dtype=np.float64)                      # [B,H,D]
        u = (qmean / np.linalg.norm(qmean, axis=-1, keepdims=True)).astype(f32)
        for bi in range(B):
            for hi in range(H):
                sel = rng.choice(nkb, size=n_shift, replace=False)
                shifted[bi, hi] = np.sort(sel)
                add = f32(w.shift_amount) * u[bi, hi]
                for j in sel:
                    k[bi, hi, j * b:min((j + 1) * b, Nk), :] += add
    out = {"workload": w, "B": B, "H": H, "D": D, "Nq": Nq, "Nk": Nk,
           "block": b, "n_forced_tokens": w.n_forced_tokens,
           "density": w.density, "dtype": w.dtype, "shifted_blocks": shifted}
    if w.dtype == "bf16":
        out["q"] = bf16_bits_from_f32(q)
        del q
        out["k"] = bf16_bits_from_f32(k)
        del k
        out["v"] = bf16_bits_from_f32(v)
        del v
    elif w.dtype == "fp32":
        out["q"], out["k"], out["v"] = q, k, v
    else:
        raise ValueError(w.dtype)
    return out
