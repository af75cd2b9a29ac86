"""The two fp64 matrix-core forms of the block-score sums give the same bits.

The score kernel forms each exact score (Eq. 2 of the SparSTAR pages: the
product of the block means, summed in float64 and rounded once) on 16 x 16
tiles of v_mfma_f64_16x16x4f64 (score_tile16); the band selection forms the
exact scores of one row on v_mfma_f64_4x4x4f64 (score_row16), with the same
four-dimension groups in the same order.  The screened selection is only
bit-identical to the two-call route if both give the same float64 sums, so
this compares them bit for bit on operands chosen to stress the rounding
(wide exponent ranges, cancelling pairs, large partial sums), through the
tests' own helper library built from the library's header.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

HELPER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libf64sums.so")


def _helper():
    assert os.path.exists(HELPER), f"{HELPER} is missing: run __graft_entry__.build()"
    lib = ctypes.CDLL(HELPER)
    lib.f64_sums_run.restype = ctypes.c_int
    lib.f64_sums_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_helper_library_exports_its_entry_point():
    lib = _helper()
    assert hasattr(lib, "f64_sums_run")


def _operands(kind, rng, cases, D):
    shape = (cases, 16, D)
    if kind == "normal":
        q, k = rng.standard_normal(shape), rng.standard_normal(shape)
    elif kind == "wide":   # magnitudes 2^-30 .. 2^30, random signs
        q = np.exp2(rng.uniform(-30, 30, shape)) * rng.choice([-1.0, 1.0], shape)
        k = np.exp2(rng.uniform(-30, 30, shape)) * rng.choice([-1.0, 1.0], shape)
    elif kind == "cancelling":   # consecutive dimensions cancel to about 2^-20
        q = rng.standard_normal(shape)
        q[:, :, 1::2] = -q[:, :, 0::2] * (1 + 2.0 ** -20 * rng.standard_normal((cases, 16, D // 2)))
        k = np.abs(rng.standard_normal(shape))
        k[:, :, 1::2] = k[:, :, 0::2]
    elif kind == "partial":   # large partial sums with sign flips, k = q * 2^[-3, 3]
        q = rng.standard_normal(shape)
        k = q * np.exp2(rng.integers(-3, 4, shape))
        k[:, :, ::3] *= -1
    else:
        raise ValueError(kind)
    return q.astype(np.float32), k.astype(np.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["normal", "wide", "cancelling", "partial"])
def test_row_form_matches_tile_form_bitwise(kind, D):
    lib = _helper()
    cases = 2048
    rng = np.random.default_rng(1000 * D + sum(map(ord, kind)))
    q, k = _operands(kind, rng, cases, D)
    dev = torch.device("cuda:0")
    Q, K = torch.from_numpy(q).to(dev), torch.from_numpy(k).to(dev)
    tile = torch.full((cases, 16, 16), float("nan"), dtype=torch.float64, device=dev)
    row = torch.full((cases, 16, 16), float("nan"), dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    rc = lib.f64_sums_run(Q.data_ptr(), K.data_ptr(), cases, D, tile.data_ptr(), row.data_ptr(),
                          stream.cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    a, b = tile.cpu().numpy(), row.cpu().numpy()
    # every sum written, and near the float64 product sum (a gross layout error fails here)
    assert np.isfinite(a).all() and np.isfinite(b).all()
    ref = np.einsum("cid,cjd->cij", q.astype(np.float64), k.astype(np.float64))
    scale = np.einsum("cid,cjd->cij", np.abs(q.astype(np.float64)), np.abs(k.astype(np.float64)))
    assert np.all(np.abs(a - ref) <= 1e-13 * scale)
    diff = int((a.view(np.uint64) != b.view(np.uint64)).sum())
    print(f"[f64 sums] {kind} D={D}: {a.size} sums, {diff} differ in any bit", flush=True)
    assert diff == 0
