"""The oracle against what the pages and the mathematics fix (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P
from workloads import make_inputs
from workloads.configs import TINY, MID, SWEEP_DENSITIES, BLOCK, L72K


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_counts_tiny_workload():
    x = make_inputs(TINY)
    q, k = oracle.decode(x["q"], "fp32"), oracle.decode(x["k"], "fp32")
    S = oracle.block_scores(oracle.block_means(q), oracle.block_means(k))
    P.pin_counts(oracle, S, 1, TINY.density)
    # offsets make the tiny rankings well separated: no near ties at the boundary
    for r in S.reshape(-1, S.shape[-1]):
        s = np.sort(r[1:])[::-1]
        assert s[3] - s[4] > 1e-4


@pytest.mark.slow
def test_counts_mid_workload():
    x = make_inputs(MID)
    q, k = oracle.decode(x["q"], "bf16"), oracle.decode(x["k"], "bf16")
    S = oracle.block_scores(oracle.block_means(q), oracle.block_means(k))
    F_ = oracle.forced_blocks(MID.n_forced_tokens)
    assert F_ == 4
    P.pin_counts(oracle, S, F_, MID.density)
    count, _ = oracle.select_blocks(S, F_, MID.density)
    assert int(count.reshape(-1)[0]) == 57


def test_pages_parameters():
    g = json.load(open(os.path.join(P.GOLDEN, "pages_parameters.json")))
    assert tuple(g["density_schedule"]["value"]) == SWEEP_DENSITIES
    assert g["block_size"]["value"] == BLOCK
    assert g["final_scale_tokens"]["value"] == L72K.Nq
    # every schedule value is dyadic, so density * E is exact in fp64
    for rho in SWEEP_DENSITIES:
        assert (rho * 2 ** 6).is_integer()
    # at the final scale's budget the 1125 eligible blocks keep 106
    assert oracle.kept_blocks(L72K.nkb, 4, SWEEP_DENSITIES[3]) == 110


def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    vals = oracle.decode(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -1.0
    assert vals[2] == 3.140625
    assert vals[3] == 2.0 ** -133
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127
