"""The screened selection's error bound, checked on the CPU by emulating the
screening arithmetic: each float32 mean split into bf16 hi + lo, the products
hi*hi + hi*lo + lo*hi accumulated in float32, scaled by tau in float32 and
stored as float16 (A), against F = the float64 dot product of the float32
means scaled by tau and rounded once to float32 (the score the two-call route
ranks).  The selection kernel claims, for every block,
    |A - F| <= e(A) = 1.001 (e1 + 6e-4 |A|),  e1 = 1.2e-4 |tau| |qbar| max|kbar| + 1e-7,
and derives from it thresholds hi > T and lo < T around T = the k-th largest A
such that A > hi forces F above F's k-th largest and A < lo below it.  These
tests check both claims on inputs chosen to stress them (cancellation,
scales far from 1, tiny and huge values, negative and zero tau); the
accumulation order here differs from the matrix core's, which the bound
covers by construction (any order)."""
import numpy as np
import pytest


def bf16_rne(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def screened(q, k, tau):
    """A [nq, nk]: the emulated screening (float32 arithmetic throughout)."""
    qh = bf16_rne(q); ql = bf16_rne(q - qh)
    kh = bf16_rne(k); kl = bf16_rne(k - kh)
    acc = np.zeros((q.shape[0], k.shape[0]), dtype=np.float32)
    # term by term, dimension by dimension, in float32 (a sequential order)
    for d in range(q.shape[1]):
        for a, b in ((qh, kh), (qh, kl), (ql, kh)):
            acc = (acc + np.outer(a[:, d], b[:, d]).astype(np.float32)).astype(np.float32)
    with np.errstate(over="ignore"):
        return (np.float32(tau) * acc).astype(np.float32).astype(np.float16).astype(np.float32)


def exact(q, k, tau):
    return (np.float64(np.float32(tau)) * (q.astype(np.float64) @ k.astype(np.float64).T)).astype(np.float32)


def bound(A, q, k, tau):
    qn = np.sqrt((q.astype(np.float64) ** 2).sum(1)) * 1.0001
    kmax = np.sqrt((k.astype(np.float64) ** 2).sum(1).max()) * 1.0001
    e1 = 1.2e-4 * abs(np.float32(tau)) * qn[:, None] * kmax + 1e-7
    return 1.001 * (e1 + 6e-4 * np.abs(A.astype(np.float64)))


def thresholds(t, e1):
    """The kernel's hi and lo for threshold t (float32 arithmetic)."""
    t, e1 = np.float32(t), np.float32(e1)
    X = t + np.float32(2.002) * e1 + np.float32(6.006e-4) * abs(t)
    Y = t - np.float32(2.002) * e1 - np.float32(6.006e-4) * abs(t)
    hi = X + np.float32(7e-4) * abs(X) + np.float32(1e-7)
    lo = Y - np.float32(7e-4) * abs(Y) - np.float32(1e-7)
    return float(hi), float(lo)


CASES = {
    "unit": lambda r, D: (r.standard_normal((24, D)) * 0.3, r.standard_normal((300, D)) * 0.3),
    "cancel": lambda r, D: (np.repeat(r.standard_normal((1, D)), 24, 0) * 3.0,
                            (lambda b: b - np.outer(b @ np.ones(D) / D, np.ones(D)))(r.standard_normal((300, D)) * 3.0)),
    "large": lambda r, D: (r.standard_normal((24, D)) * 40.0, r.standard_normal((300, D)) * 40.0),
    "tiny": lambda r, D: (r.standard_normal((24, D)) * 1e-3, r.standard_normal((300, D)) * 1e-3),
    "offset": lambda r, D: (r.standard_normal((24, D)) + 2.0, r.standard_normal((300, D)) * 0.2 + 1.0),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("tau_sign", [1.0, -1.0])
def test_screened_values_stay_within_the_bound(case, D, tau_sign):
    r = np.random.default_rng(sum(map(ord, case)) * 1000 + D)   # deterministic per case
    q, k = (a.astype(np.float32) for a in CASES[case](r, D))
    tau = tau_sign / np.sqrt(D)
    A, F = screened(q, k, tau), exact(q, k, tau)
    ok = np.isfinite(A)
    assert ok.any()
    err = np.abs(A.astype(np.float64) - F.astype(np.float64))
    e = bound(A, q, k, tau)
    assert np.all(err[ok] <= e[ok]), float((err[ok] / e[ok]).max())
    # the bound is not vacuous: the worst case uses a visible share of it
    assert (err[ok] / e[ok]).max() > 1e-3


@pytest.mark.parametrize("case", sorted(CASES))
def test_thresholds_keep_and_drop_only_what_the_exact_scores_decide(case):
    D, kfrac = 128, 0.1
    r = np.random.default_rng(7 + len(case))
    q, k = (a.astype(np.float32) for a in CASES[case](r, D))
    tau = 1 / np.sqrt(D)
    A, F = screened(q, k, tau), exact(q, k, tau)
    qn = np.sqrt((q.astype(np.float64) ** 2).sum(1)) * 1.0001
    kmax = np.sqrt((k.astype(np.float64) ** 2).sum(1).max()) * 1.0001
    kk = int(np.ceil(kfrac * k.shape[0]))
    checked = 0
    for i in range(q.shape[0]):
        a, f = A[i], F[i]
        if not np.all(np.isfinite(a)):
            continue
        t = np.sort(a)[::-1][kk - 1]
        f_k = np.sort(f)[::-1][kk - 1]
        e1 = 1.2e-4 * abs(tau) * qn[i] * kmax + 1e-7
        e_t = 1.001 * (e1 + 6e-4 * abs(t))
        assert t - e_t <= f_k <= t + e_t
        hi, lo = thresholds(t, e1)
        assert lo < t < hi
        assert np.all(f[a > hi] > f_k)       # kept without an exact score
        assert np.all(f[a < lo] < f_k)       # dropped without an exact score
        checked += 1
    assert checked == q.shape[0]


@pytest.mark.parametrize("case,term", [("offset", "storage"), ("large", "computation"),
                                       ("unit", "computation")])
def test_both_terms_of_the_bound_are_needed(case, term):
    """Dropping either term of e(A) makes the first check fail on these
    inputs: the float16 storage term (relative to |A|, large where the scores
    are large) and the computation term e1 (where |A| is small against
    |tau| |qbar| max|kbar|)."""
    r = np.random.default_rng(5)
    q, k = (a.astype(np.float32) for a in CASES[case](r, 128))
    tau = 1 / np.sqrt(128)
    A, F = screened(q, k, tau), exact(q, k, tau)
    ok = np.isfinite(A)
    err = np.abs(A.astype(np.float64) - F.astype(np.float64))[ok]
    qn = np.sqrt((q.astype(np.float64) ** 2).sum(1)) * 1.0001
    kmax = np.sqrt((k.astype(np.float64) ** 2).sum(1).max()) * 1.0001
    e1 = (1.2e-4 / np.sqrt(128) * qn[:, None] * kmax + 1e-7) * np.ones_like(A, dtype=np.float64)
    if term == "storage":
        assert np.any(err > 1.001 * e1[ok])
    else:
        assert np.any(err > 1.001 * (6e-4 * np.abs(A.astype(np.float64)[ok]) + 1e-7))
