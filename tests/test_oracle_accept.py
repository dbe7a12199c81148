"""Pins for the oracle's acceptance rules (CPU only).

Greedy: brute force over forced drafts for every k, the Figure 1(c) case,
lowest-id ties.  Rejection sampling: the first emitted token's distribution
equals the target's, measured exactly by locating the oracle's own decision
boundaries in (r_1, r*) by bisection (no formula restated), plus a seeded
Monte-Carlo chi-square test, q = p (always accept) and disjoint supports
(always reject, correction drawn from p).
"""
import json
import os

import numpy as np
import pytest
import scipy.stats

from oracle import accept_candidates, greedy_accept, rejection_accept

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _peaked_logits(r, V, tokens):
    """rows whose unique argmax is the given token (N(0,2) elsewhere)."""
    z = r.normal(0, np.sqrt(2), (len(tokens), V)).astype(np.float32)
    for i, t in enumerate(tokens):
        z[i, t] = z[i].max() + 1.0
    return z


@pytest.mark.parametrize("gamma", [1, 6, 12])
def test_greedy_every_k(gamma):
    r = np.random.default_rng(gamma)
    V = 512
    for k in range(gamma + 1):
        g = r.integers(0, V, gamma + 1)              # target argmax per row
        drafts = g[:gamma].copy()
        if k < gamma:
            drafts[k] = (g[k] + 1 + r.integers(0, V - 1)) % V   # first mismatch at draft k+1
            drafts[k + 1:] = r.integers(0, V, gamma - k - 1)
        zt = _peaked_logits(r, V, g)
        kk, nxt, margin = greedy_accept(zt, drafts)
        assert kk == k
        assert nxt == g[k]            # correction (k < gamma) or bonus (k == gamma)
        assert margin > 0.5


def test_greedy_ties_lowest_id():
    zt = np.zeros((3, 8), np.float32)
    zt[0, [2, 5]] = 1.0
    zt[1, [1, 3]] = 2.0
    k, nxt, margin = greedy_accept(zt, np.array([2, 3]))
    assert (k, nxt, margin) == (1, 1, 0.0)


def test_fig1_worked_example_acceptance():
    """EvSpark Figure 1(c): six drafts, three accepted, correction becomes the next anchor."""
    with open(os.path.join(GOLDEN, "fig1_worked_example.json")) as fh:
        fx = json.load(fh)
    gamma, acc = fx["gamma"], fx["accepted"]
    r = np.random.default_rng(61)
    g = r.integers(0, 512, gamma + 1)
    drafts = g[:gamma].copy()
    drafts[acc] = (g[acc] + 7) % 512
    k, nxt, _ = greedy_accept(_peaked_logits(r, 512, g), drafts)
    assert k == acc
    assert nxt == g[acc] and nxt != drafts[acc]
    assert fx["emitted_per_round"] == k + 1


# ------------------------------------------------------------ rejection sampling

def _boundary(f, lo, hi, iters=80):
    """Bisect the point where the step function f changes value in [lo, hi)."""
    flo = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) == flo:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _exact_first_token_distribution(zt, zd, V):
    """P(first emitted token = t) for gamma = 1, integrating the oracle over (r_1, r*) exactly.

    For each draft t1 (probability q(t1)) the oracle's accept decision is a
    step in r_1 and its resampled token a monotone step function of r*; both
    boundaries are located by bisection on the oracle itself.
    """
    q = _softmax(zd[0].astype(np.float64))
    dist = np.zeros(V)
    for t1 in range(V):
        drafts = np.array([t1])
        acc = lambda r1: rejection_accept(zt, zd, drafts, np.array([r1, 0.5]))[0]
        if acc(0.0) == 0:
            a = 0.0
        elif acc(1.0 - 1e-16) == 1:
            a = 1.0
        else:
            a = _boundary(acc, 0.0, 1.0 - 1e-16)
        dist[t1] += q[t1] * a
        if a < 1.0:
            r1 = min(1.0 - 1e-16, a + (1.0 - a) / 2)          # any r_1 in the reject region
            tok = lambda rs: rejection_accept(zt, zd, drafts, np.array([r1, rs]))[1]
            edges = [0.0]
            cur = 0.0
            while tok(cur) != tok(1.0 - 1e-16):
                nxt_edge = _boundary(tok, cur, 1.0 - 1e-16)
                dist[tok(cur)] += q[t1] * (1.0 - a) * (nxt_edge - edges[-1])
                edges.append(nxt_edge)
                cur = nxt_edge + 1e-15
            dist[tok(1.0 - 1e-16)] += q[t1] * (1.0 - a) * (1.0 - edges[-1])
    return dist


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rejection_first_token_is_target_distributed_exactly(seed):
    r = np.random.default_rng(seed)
    V = 4
    zt = r.normal(0, np.sqrt(2), (2, V)).astype(np.float32)
    zd = r.normal(0, np.sqrt(2), (1, V)).astype(np.float32)
    dist = _exact_first_token_distribution(zt, zd, V)
    np.testing.assert_allclose(dist, _softmax(zt[0].astype(np.float64)), atol=1e-9)


def test_rejection_pin_catches_wrong_residual(monkeypatch):
    """A planted mistake in the oracle (|p - q| instead of max(0, p - q)) breaks the pin."""
    import oracle.acceptance as acc_mod
    r = np.random.default_rng(5)
    V = 4
    zt = r.normal(0, np.sqrt(2), (2, V)).astype(np.float32)
    zd = r.normal(0, np.sqrt(2), (1, V)).astype(np.float32)
    monkeypatch.setattr(acc_mod, "np", _NumpyWithoutClamp())
    dist = _exact_first_token_distribution(zt, zd, V)
    monkeypatch.undo()
    assert np.max(np.abs(dist - _softmax(zt[0].astype(np.float64)))) > 1e-3


class _NumpyWithoutClamp:
    """numpy, except that max(0, p - q) keeps the negative part (a dropped clamp)."""
    def __getattr__(self, name):
        if name == "maximum":
            return lambda a, b: np.abs(np.asarray(b, dtype=np.float64)) if np.isscalar(a) else np.maximum(a, b)
        return getattr(np, name)


def test_rejection_monte_carlo_chi_square():
    """Over seeded rounds the first two emitted tokens follow p_0 and (given acceptance) p_1."""
    r = np.random.default_rng(12)
    V, gamma, n = 6, 2, 20000
    zt = r.normal(0, np.sqrt(2), (gamma + 1, V)).astype(np.float32)
    zd = r.normal(0, np.sqrt(2), (gamma, V)).astype(np.float32)
    qs = [_softmax(zd[i].astype(np.float64)) for i in range(gamma)]
    first = np.zeros(V)
    second = np.zeros(V)
    for _ in range(n):
        drafts = np.array([r.choice(V, p=qs[i]) for i in range(gamma)])
        u = r.random(gamma + 1)
        k, nxt, _ = rejection_accept(zt, zd, drafts, u)
        emitted = list(drafts[:k]) + [nxt]
        first[emitted[0]] += 1
        if len(emitted) > 1:
            second[emitted[1]] += 1
    for counts, row in ((first, 0), (second, 1)):
        p = _softmax(zt[row].astype(np.float64))
        stat, pval = scipy.stats.chisquare(counts, counts.sum() * p)
        assert pval > 1e-4, (row, counts, p)


def test_rejection_q_equals_p_accepts_everything():
    r = np.random.default_rng(13)
    V, gamma = 512, 12
    z = r.normal(0, np.sqrt(2), (gamma + 1, V)).astype(np.float32)
    for trial in range(20):
        drafts = r.integers(0, V, gamma)
        u = r.random(gamma + 1)
        # draft i is drawn from the same distribution the target assigns it: ratio 1 > r
        k, _, _ = rejection_accept(z, z[:gamma], drafts, u)
        assert k == gamma


def test_rejection_disjoint_supports_reject_and_correct_from_p():
    V, gamma = 8, 3
    zt = np.full((gamma + 1, V), -1e4, np.float32)
    zd = np.full((gamma, V), -1e4, np.float32)
    zt[:, :4] = np.array([0.0, 1.0, -0.5, 0.3], np.float32)    # target mass on tokens 0..3
    zd[:, 4:] = 0.0                                             # drafts only from 4..7
    p0 = _softmax(zt[0].astype(np.float64))
    cdf = np.cumsum(p0)
    r = np.random.default_rng(14)
    for _ in range(50):
        drafts = r.integers(4, 8, gamma)
        u = r.random(gamma + 1)
        k, nxt, _ = rejection_accept(zt, zd, drafts, u)
        assert k == 0
        assert nxt == int(np.searchsorted(cdf, u[gamma] * cdf[-1], side="right"))


def test_multi_candidate_winner_lowest_on_ties():
    r = np.random.default_rng(15)
    V, gamma, nb, nc = 64, 4, 2, 4
    g = r.integers(0, V, (nb, nc, gamma + 1))
    zt = np.stack([np.stack([_peaked_logits(r, V, g[b, c]) for c in range(nc)]) for b in range(nb)])
    drafts = g[:, :, :gamma].copy()
    want = [[1, 3, 3, 0], [2, 2, 1, 2]]
    for b in range(nb):
        for c in range(nc):
            kk = want[b][c]
            if kk < gamma:
                drafts[b, c, kk] = (g[b, c, kk] + 1) % V
    n_acc, nxt, best, _ = accept_candidates("greedy", zt, None, drafts, None)
    np.testing.assert_array_equal(n_acc, want)
    np.testing.assert_array_equal(best, [1, 0])
