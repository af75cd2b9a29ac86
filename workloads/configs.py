"""The five benchmark workloads, by name and size.

Key sequences follow the visible-context order of InfinityStar's SSA attention
as the SparSTAR review lists it under "Assumptions & free parameters" (Eq. 1):
text tokens, then the reference (preceding clip's final scale, or for Clip 1
the final image-pyramid reference), then the current scale.  The forced
(always-dense) context is therefore a token prefix of the key sequence.

Density values come from the schedule the review gives under "What carries
the argument" and "free parameters" (0.625, 0.1875, 0.1875, 0.09375 over the
four sparsified scales); the block size of 128 tokens is one of the
review's free parameters.  The 72,000-token final scale is
named in "What carries the argument".
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

BLOCK = 128
TEXT_TOKENS = 512


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    dtype: str              # "fp32" or "bf16" (storage and compute input type)
    Nq: int                 # current-scale query tokens
    n_text: int             # text tokens (forced)
    n_ref: int              # reference tokens
    ref_forced: bool        # True for Clip 1's image-pyramid reference
    n_cur: int              # current-scale key tokens
    density: float
    block: int = BLOCK
    # value recipe
    offset_std: float = 0.3         # per-block mean offsets
    offset_q: bool = True           # offsets on Q blocks
    offset_v: bool = True           # offsets on V blocks
    shift_frac: float = 0.05        # fraction of key blocks shifted along the query mean
    shift_amount: float = 1.0
    seed: int = 0
    # Explicit forced-token count; None derives it from the segments.
    forced_tokens_override: Optional[int] = None

    @property
    def Nk(self) -> int:
        return self.n_text + self.n_ref + self.n_cur

    @property
    def n_forced_tokens(self) -> int:
        if self.forced_tokens_override is not None:
            return self.forced_tokens_override
        return self.n_text + (self.n_ref if self.ref_forced else 0)

    @property
    def nqb(self) -> int:
        return -(-self.Nq // self.block)

    @property
    def nkb(self) -> int:
        return -(-self.Nk // self.block)

    def with_density(self, density: float) -> "Workload":
        return Workload(**{**self.__dict__, "density": density,
                           "name": f"{self.name}@rho={density:g}"})

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "D": self.D,
                "dtype": self.dtype, "Nq": self.Nq, "Nk": self.Nk,
                "n_text": self.n_text, "n_ref": self.n_ref,
                "ref_forced": self.ref_forced, "n_cur": self.n_cur,
                "n_forced_tokens": self.n_forced_tokens,
                "density": self.density, "block": self.block, "seed": self.seed}


# 0: tiny CPU-checkable case.  2048 queries, 2048 keys; block 0 is text.
TINY = Workload(name="tiny-2k-fp32", B=1, H=1, D=64, dtype="fp32", Nq=2048,
                n_text=128, n_ref=0, ref_forced=False, n_cur=1920,
                density=0.25, offset_std=0.5, offset_q=False, offset_v=False,
                shift_frac=0.0)
# 1: mid refinement scale, one attention layer.
MID = Workload(name="mid-18k", B=1, H=16, D=128, dtype="bf16", Nq=18000,
               n_text=TEXT_TOKENS, n_ref=18000, ref_forced=False, n_cur=18000,
               density=0.1875)
# 2: the 72,000-token final scale.
L72K = Workload(name="final-72k", B=1, H=16, D=128, dtype="bf16", Nq=72000,
                n_text=TEXT_TOKENS, n_ref=72000, ref_forced=False, n_cur=72000,
                density=0.09375)
# 3: Clip-1 variant: text + 3,600-token image-pyramid reference, both forced.
CLIP1 = Workload(name="clip1-72k", B=1, H=16, D=128, dtype="bf16", Nq=72000,
                 n_text=TEXT_TOKENS, n_ref=3600, ref_forced=True, n_cur=72000,
                 density=0.09375)

SWEEP_SCALES: Tuple[int, ...] = (8000, 18000, 32000, 72000)
SWEEP_DENSITIES: Tuple[float, ...] = (0.625, 0.1875, 0.1875, 0.09375)


def sweep_workloads(dense: bool = False):
    """4: the four-scale sweep, batch 2, each scale with a matching reference."""
    out = []
    for n, rho in zip(SWEEP_SCALES, SWEEP_DENSITIES):
        out.append(Workload(name=f"sweep-{n // 1000}k" + ("-dense" if dense else ""),
                            B=2, H=16, D=128, dtype="bf16", Nq=n,
                            n_text=TEXT_TOKENS, n_ref=n, ref_forced=False, n_cur=n,
                            density=1.0 if dense else rho))
    return out


CONFIGS = {
    0: [TINY],
    1: [MID],
    2: [L72K],
    3: [CLIP1],
    4: sweep_workloads(False) + sweep_workloads(True),
}


def workload(name: str) -> Workload:
    for ws in CONFIGS.values():
        for w in ws:
            if w.name == name:
                return w
    raise KeyError(name)
