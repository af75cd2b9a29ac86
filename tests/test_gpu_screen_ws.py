"""The screened scores themselves, read back from the workspace (white-box).

sparstar_select_blocks_from_means first screens every block score on the
bf16 matrix cores (hi/lo split of the float32 means), stores it as float16
in its workspace together with the largest squared key-block norm of each
strip of 128 blocks, and then decides the blocks near each row's k-th largest
on exact scores.  The selection tests check the end result; this checks the
intermediate the correctness argument rests on, against the exact scores of
Eq. 2 (SparSTAR pages, Pith review, "What carries the argument") in float64:

* every screened value A of an eligible block lies within
  e(A) = 1.001 (1.2e-4 |tau| |qbar_i| max_j |kbar_j| + 1e-7 + 6e-4 |A|)
  of F = float32(tau * qbar_i . kbar_j) -- the bound the band selection uses
  (with the true norms, which the library only ever rounds upwards);
* forced blocks and the slots past nkb hold the sentinel 0xffff;
* the strip maxima are the largest squared norms, to float32 rounding.

Workspace layout (the library's, not part of its contract): float16
[B*H][nqb][128 * ceil(nkb / 128)], then at the next 256-byte boundary
float32 [B*H][ceil(nkb / 128)].
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_head_amd as sp
from tests.parity_util import log

pytestmark = pytest.mark.gpu

CASES = [
    # D, nqb, nkb, F, density, kind
    (128, 37, 1129, 4, 0.09375, "normal"),
    (64, 33, 1129, 4, 0.09375, "normal"),
    (128, 20, 300, 0, 0.5, "normal"),
    (128, 9, 65, 65, 0.5, "normal"),          # every block forced
    (128, 33, 1129, 4, 0.09375, "scaled"),    # means far from unit scale
    (128, 18, 300, 4, 0.5, "neg_tau"),
    (64, 17, 2048, 33, 0.2, "wide"),          # element magnitudes over 12 binades
    (128, 5, 129, 1, 0.3, "normal"),          # one block past a strip
]


def _means(D, nqb, nkb, kind, seed):
    rng = np.random.default_rng(seed)
    qb = (rng.standard_normal((2, 2, nqb, D)) * 0.3).astype(np.float32)
    kb = (rng.standard_normal((2, 2, nkb, D)) * 0.3).astype(np.float32)
    if kind == "scaled":
        qb = (qb * 3e3).astype(np.float32)
        kb = (kb * 2e-3).astype(np.float32)
    elif kind == "wide":
        # (kept inside the float16 range of the screened values)
        qb = (qb * np.exp2(rng.uniform(-6, 6, qb.shape))).astype(np.float32)
        kb = (kb * np.exp2(rng.uniform(-6, 6, kb.shape))).astype(np.float32)
    return qb, kb


@pytest.mark.parametrize("D,nqb,nkb,F,density,kind", CASES)
def test_screened_scores_within_the_bound(D, nqb, nkb, F, density, kind):
    log(f"screened scores D={D} nqb={nqb} nkb={nkb} F={F} kind={kind}")
    qb, kb = _means(D, nqb, nkb, kind, seed=nqb * 31 + nkb + D)
    tau = -1.0 / math.sqrt(D) if kind == "neg_tau" else 1.0 / math.sqrt(D)
    B, H = qb.shape[:2]
    BH = B * H
    dev = torch.device("cuda:0")
    ws = sp.select_workspace(B, H, nqb, nkb, dev)
    ws.fill_(0x5a)                       # stale bytes: everything read must be written
    sp.select_blocks_from_means(torch.from_numpy(qb).to(dev), torch.from_numpy(kb).to(dev), F,
                                density, tau=tau, workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()

    cstrips = -(-nkb // 128)
    stride = 128 * cstrips
    kmax_off = -(-(BH * nqb * stride * 2) // 256) * 256
    assert raw.size >= kmax_off + BH * cstrips * 4
    A16 = raw[:BH * nqb * stride * 2].view(np.uint16).reshape(BH, nqb, stride)
    kmaxp = raw[kmax_off:kmax_off + BH * cstrips * 4].view(np.float32).reshape(BH, cstrips)

    q64 = qb.reshape(BH, nqb, D).astype(np.float64)
    k64 = kb.reshape(BH, nkb, D).astype(np.float64)
    # strip maxima of the squared key norms (rows past nkb repeat the last block)
    n2 = (k64 ** 2).sum(axis=-1)
    for s in range(cstrips):
        ref = n2[:, 128 * s:min(128 * s + 128, nkb)].max(axis=1)
        got = kmaxp[:, s].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 2e-5 * ref + 1e-30), (s, got, ref)

    # sentinels: forced blocks and slots past nkb
    assert np.all(A16[:, :, :F] == 0xffff)
    assert np.all(A16[:, :, nkb:] == 0xffff)

    # eligible blocks: |A - F| <= e(A)
    tau32 = float(np.float32(tau))                              # the float the library receives
    S64 = tau32 * np.einsum("bid,bjd->bij", q64, k64)
    Fv = S64.astype(np.float32).astype(np.float64)[:, :, F:]
    A = A16[:, :, F:nkb].view(np.float16).astype(np.float64)
    assert np.isfinite(A).all()
    qn = np.sqrt((q64 ** 2).sum(axis=-1))                       # [BH, nqb]
    kmax = np.sqrt(n2.max(axis=1))                              # [BH]
    e1 = 1.2e-4 * abs(tau32) * qn * kmax[:, None] + 1e-7
    e = 1.001 * (e1[:, :, None] + 6e-4 * np.abs(A))
    err = np.abs(A - Fv)
    worst = float((err / e).max()) if err.size else 0.0
    log(f"  {A.size} screened values, worst |A - F| / e(A) = {worst:.3f}")
    assert np.all(err <= e)
