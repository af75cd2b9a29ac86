"""The seeded input generator: determinism, shapes, sizes, rounding (CPU only)."""
import numpy as np
import pytest

from workloads import make_inputs, bf16_bits_from_f32, CONFIGS
from workloads.configs import TINY, MID, L72K, CLIP1, sweep_workloads


def test_block_counts():
    assert (TINY.nqb, TINY.nkb, TINY.n_forced_tokens) == (16, 16, 128)
    assert (MID.Nk, MID.nqb, MID.nkb) == (36512, 141, 286)
    assert (L72K.Nk, L72K.nqb, L72K.nkb) == (144512, 563, 1129)
    assert (CLIP1.Nk, CLIP1.nkb, CLIP1.n_forced_tokens) == (76112, 595, 4112)
    sw = sweep_workloads()
    assert [w.nkb for w in sw] == [129, 286, 504, 1129]
    assert [w.density for w in sweep_workloads(True)] == [1.0] * 4
    assert len(CONFIGS) == 5


def test_bf16_rounding():
    # halfway cases round to even; values above half round up
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 1.5 * 2 ** -8, -2.5, 0.0, -0.0],
                 dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000]
    # against torch's own cast
    import torch
    y = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    tb = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(y), tb)


def test_deterministic_and_shapes():
    a = make_inputs(TINY)
    b = make_inputs(TINY)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (1, 1, 2048, 64) and a["q"].dtype == np.float32
    c = make_inputs(TINY, seed=1)
    assert not np.array_equal(a["q"], c["q"])


def test_tiny_offsets_on_keys_only():
    x = make_inputs(TINY)
    kb = x["k"][0, 0].reshape(16, 128, 64).mean(axis=1)
    qb = x["q"][0, 0].reshape(16, 128, 64).mean(axis=1)
    # key block means spread with the 0.5 offsets; query block means are ~N(0, 1/128)
    assert 0.4 < kb.std() < 0.6
    assert qb.std() < 0.15


@pytest.mark.slow
def test_mid_shapes_and_shift():
    x = make_inputs(MID)
    assert x["q"].shape == (1, 16, 18000, 128) and x["q"].dtype == np.uint16
    assert x["k"].shape == (1, 16, 36512, 128)
    assert x["shifted_blocks"].shape == (1, 16, 14)
    for h in range(16):
        assert len(set(x["shifted_blocks"][0, h])) == 14
