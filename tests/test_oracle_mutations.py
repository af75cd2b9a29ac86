"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

A mutation is a textual edit of the oracle's source; the edited copy is loaded
as a fresh module (on the CPU only) and every pin is run against it.  At least
one pin must fail for every mutation, otherwise the pins leave that part of the
oracle unchecked.
"""
import inspect
import types

import pytest

import oracle.sparstar_oracle as O
from tests import oracle_pins as P

MUTATIONS = {
    "score-drops-tau": ("S[..., i0:i1, :] = tau * prod.sum(axis=-1)",
                        "S[..., i0:i1, :] = prod.sum(axis=-1)"),
    "score-tau-inverted": ("tau = 1.0 / math.sqrt(D)", "tau = math.sqrt(D)"),
    "mean-divides-by-block": ("out[..., i, :] = x[..., lo:hi, :].sum(axis=-2) / (hi - lo)",
                              "out[..., i, :] = x[..., lo:hi, :].sum(axis=-2) / block"),
    "mean-drops-last-token": ("x[..., lo:hi, :].sum(axis=-2) / (hi - lo)",
                              "x[..., lo:max(lo + 1, hi - 1), :].sum(axis=-2) / (hi - lo)"),
    "budget-floor": ("return int(math.ceil(float(density) * float(n_eligible)))",
                     "return int(math.floor(float(density) * float(n_eligible)))"),
    "budget-over-all-blocks": ("k = budget(eligible.size, density)", "k = budget(nkb, density)"),
    "forced-floor": ("return -(-int(n_forced_tokens) // block)", "return int(n_forced_tokens) // block"),
    "ranks-ascending": ("order = np.argsort(-s_row[n_forced:], kind=\"stable\")",
                        "order = np.argsort(s_row[n_forced:], kind=\"stable\")"),
    "ties-to-higher-index": ("order = np.argsort(-s_row[n_forced:], kind=\"stable\")",
                             "order = (nkb - n_forced - 1) - np.argsort(-s_row[n_forced:][::-1], kind=\"stable\")"),
    "forced-not-kept": ("return np.sort(np.concatenate([np.arange(n_forced), top]))",
                        "return np.sort(top)"),
    "index-unsorted": ("return np.sort(np.concatenate([np.arange(n_forced), top]))",
                       "return np.concatenate([np.arange(n_forced), top])"),
    "attn-no-scale": ("logits = scale * (q_blk @ k[keys].T)", "logits = (q_blk @ k[keys].T)"),
    "attn-values-are-keys": ("o = (e / z) @ v[keys]", "o = (e / z) @ k[keys]"),
    "attn-drops-partial-key-block": ("np.arange(j * block, min((j + 1) * block, Nk))",
                                     "np.arange(j * block, min((j + 1) * block, Nk - Nk % block or Nk))"),
    "lse-drops-max": ("lse = m[:, 0] + np.log(z[:, 0])", "lse = np.log(z[:, 0])"),
    "softmax-unnormalised": ("o = (e / z) @ v[keys]", "o = e @ v[keys]"),
    "empty-row-nonzero": ("return np.zeros((n, v.shape[1])), np.full(n, -np.inf)",
                          "return np.zeros((n, v.shape[1])), np.zeros(n)"),
    "mass-normalised-over-kept": ("return e / e.sum(axis=1, keepdims=True)",
                                  "return e / e[:, :1].sum(axis=1, keepdims=True)"),
    "mass-skips-last-key-of-block": ("keep[j * block:min((j + 1) * block, Nk)] = True",
                                     "keep[j * block:min((j + 1) * block, Nk) - 1] = True"),
    "bound-takes-least-probable": ("elig = np.sort(p[:, f_tok:], axis=1)[:, ::-1]",
                                   "elig = np.sort(p[:, f_tok:], axis=1)"),
    "bound-ignores-forced": ("out[(b, h, i)] = forced + elig[:, :m_tok].sum(axis=1)",
                             "out[(b, h, i)] = elig[:, :m_tok].sum(axis=1)"),
    "transfer-centre-off-by-half": ("return Fraction(first + last + 1, 2)", "return Fraction(first + last, 2)"),
    "transfer-block-start-not-centre": ("return Fraction(first + last + 1, 2)", "return Fraction(first)"),
    "transfer-source-start-not-advanced": ("            start_src += src[seg]\n", "            start_src += dst[seg]\n"),
    "transfer-relative-to-source-length": ("rel = (c - start_dst) / dst[seg]", "rel = (c - start_dst) / src[seg]"),
    "transfer-query-map-target-size": ("out[i] = math.floor(rel * src_n_cur) // block",
                                       "out[i] = math.floor(rel * dst_n_cur) // block"),
    "transfer-query-rounds-up": ("out[i] = math.floor(rel * src_n_cur) // block",
                                 "out[i] = math.ceil(rel * src_n_cur) // block"),
    "transfer-transposed-gather": ("return S_src[..., qmap[:, None], kmap[None, :]]",
                                   "return S_src[..., qmap[:, None], kmap[None, :]][..., ::-1]"),
    "flops-counts-padding": ("nk = int(np.minimum((blocks + 1) * block, Nk).sum() - (blocks * block).sum())",
                             "nk = int(blocks.size * block)"),
}


def _mutant(old, new):
    src = inspect.getsource(O)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} not caught by any pin"


def test_unmutated_source_passes():
    mod = _mutant("import math", "import math")
    for pin in P.ALL_PINS:
        pin(mod)
