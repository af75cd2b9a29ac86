"""Host-side logic of bench.py (no GPU): the one-GPU guard, the FLOP count and
the selection stage's algorithmic bytes."""
import os
import subprocess
import sys

import numpy as np

import oracle
from workloads.configs import L72K, MID, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_selected_flops_matches_oracle_count():
    rng = np.random.default_rng(3)
    for Nq, Nk, D in [(300, 700, 64), (256, 1000, 128), (129, 129, 128)]:
        nqb, nkb = -(-Nq // 128), -(-Nk // 128)
        kept = min(4, nkb)
        cnt = rng.integers(0, kept + 1, size=(2, 3, nqb)).astype(np.int32)
        idx = np.full((2, 3, nqb, kept + 1), -1, dtype=np.int32)
        for r in np.ndindex(2, 3, nqb):
            idx[r][:cnt[r]] = np.sort(rng.choice(nkb, size=cnt[r], replace=False))
        idx[0, 0, 0, -1] = nkb + 3          # past the count: never counted
        assert bench.selected_flops(cnt, idx, Nq, Nk, D) == oracle.selected_flops(cnt, idx, Nq, Nk, D)


def test_stage_bytes_closed_form():
    # Q + K read once, means written and read back, index lists written
    assert bench.stage_bytes(L72K, 110, 563, 1129) == 918_554_432
    w = MID
    nqb, nkb = -(-w.Nq // 128), -(-w.Nk // 128)
    expect = (w.Nq + w.Nk) * w.D * 2 * w.H + 2 * w.H * (nqb + nkb) * w.D * 4 + w.H * nqb * (4 * 57 + 4)
    assert bench.stage_bytes(w, 57, nqb, nkb) == expect
    assert bench.stage_bytes(TINY, 5, 16, 16) == (2048 + 2048) * 64 * 4 + 2 * 32 * 64 * 4 + 16 * 24
