"""Pins for the oracle's recursive multi-candidate acceptance (CPU only).

* one candidate: identical to the one-candidate rejection rule (itself pinned);
* the first emitted token is distributed exactly as the target's, summed over
  every combination of independent draft tokens, with the oracle's own
  decision boundaries located by bisection (no formula restated);
* planted mistakes in the residual update break that identity;
* Monte Carlo: under a toy target and drafter whose distributions depend on
  the prefix, the first two emitted tokens follow the target's joint law;
* q = p keeps every draft of the first candidate.
"""
import itertools

import numpy as np
import pytest
import scipy.stats

import oracle.acceptance as acc_mod
from oracle import accept_candidates, recursive_accept, rejection_accept

EPS1 = 1.0 - 1e-16


def _softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("gamma,V,T", [(0, 7, 1.0), (1, 3, 1.0), (6, 512, 0.5), (12, 512, 2.0), (12, 40, 1.0)])
def test_one_candidate_is_the_rejection_rule(gamma, V, T):
    r = np.random.default_rng(gamma * 100 + V)
    for trial in range(30):
        zt = r.normal(0, np.sqrt(2), (1, gamma + 1, V)).astype(np.float32)
        zd = r.normal(0, np.sqrt(2), (1, gamma, V)).astype(np.float32)
        if trial % 3 == 0 and gamma:
            zd[0, : gamma // 2] = zt[0, : gamma // 2]            # long accepted runs too
        drafts = np.stack([[r.choice(V, p=_softmax(zd[0, i] / T)) for i in range(gamma)]]).astype(np.int32)
        u = r.random((1, gamma + 1))
        n_acc, nxt, best, marg = recursive_accept(zt, zd, drafts, u, T)
        k, t, m = rejection_accept(zt[0], zd[0], drafts[0], u[0], T)
        assert (int(n_acc[0]), int(nxt), int(best)) == (k, t, 0)
        assert marg[0] == m


def _boundary(f, lo, hi, iters=80):
    flo = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) == flo:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _accept_fraction(f):
    """Measure of r in [0, 1) with f(r) true, for f true below a threshold and false above."""
    if not f(0.0):
        return 0.0
    if f(EPS1):
        return 1.0
    return _boundary(f, 0.0, EPS1)


def _draw_measure(tok, dist, weight):
    """Add weight x (measure of r* giving token y) to dist[y] for a monotone step function tok(r*)."""
    cur, left = 0.0, 0.0
    while tok(cur) != tok(EPS1):
        edge = _boundary(tok, cur, EPS1)
        dist[tok(cur)] += weight * (edge - left)
        left = edge
        cur = edge + 1e-15
    dist[tok(EPS1)] += weight * (1.0 - left)


def _exact_first_token(zt, zd, nc, V):
    """P(first emitted token = y), gamma = 1, every candidate row equal, drafts i.i.d. from q."""
    q = _softmax(zd[0, 0])
    dist = np.zeros(V)
    for combo in itertools.product(range(V), repeat=nc):
        drafts = np.array(combo, np.int32).reshape(nc, 1)
        prob = float(np.prod([q[x] for x in combo]))
        reach = 1.0
        for c in range(nc):
            def accepted(r, c=c):
                u = np.full((nc, 2), 0.5)
                u[:c, 0] = EPS1
                u[c, 0] = r
                u[c + 1:, 0] = EPS1
                n_acc, _, best, _ = recursive_accept(zt, zd, drafts, u)
                return int(n_acc[best]) >= 1 and int(best) == c
            a = _accept_fraction(accepted)
            dist[combo[c]] += prob * reach * a
            reach *= 1.0 - a
            if reach == 0.0:
                break
        if reach > 0.0:
            def tok(rs):
                u = np.full((nc, 2), EPS1)
                u[0, 1] = rs
                return int(recursive_accept(zt, zd, drafts, u)[1])
            _draw_measure(tok, dist, prob * reach)
    return dist


def _shared_rows(r, nc, V):
    zt1 = r.normal(0, np.sqrt(2), (2, V)).astype(np.float32)
    zd1 = r.normal(0, np.sqrt(2), (1, V)).astype(np.float32)
    return np.broadcast_to(zt1, (nc, 2, V)).copy(), np.broadcast_to(zd1, (nc, 1, V)).copy()


@pytest.mark.parametrize("nc,V,seed", [(2, 3, 0), (2, 4, 1), (3, 3, 2), (4, 3, 3)])
def test_first_token_is_target_distributed_exactly(nc, V, seed):
    zt, zd = _shared_rows(np.random.default_rng(seed), nc, V)
    dist = _exact_first_token(zt, zd, nc, V)
    np.testing.assert_allclose(dist, _softmax(zt[0, 0]), atol=1e-9)


@pytest.mark.parametrize("plant", ["no_update", "unnormalised"])
def test_pin_catches_planted_residual_mistakes(monkeypatch, plant):
    """A residual that is never updated, or one tested without its total, breaks the identity."""
    zt, zd = _shared_rows(np.random.default_rng(7), 3, 3)
    if plant == "no_update":
        monkeypatch.setattr(acc_mod, "_residual", lambda w, z, q: (w, z))
    else:
        monkeypatch.setattr(acc_mod, "_residual", lambda w, z, q: (np.maximum(0.0, w - q), 1.0))
    dist = _exact_first_token(zt, zd, 3, 3)
    monkeypatch.undo()
    assert np.max(np.abs(dist - _softmax(zt[0, 0]))) > 1e-3


class _ToyModel:
    """Target and drafter whose next-token logits are a seeded function of the whole prefix."""

    def __init__(self, V, seed, scale):
        self.V, self.seed, self.scale, self.memo = V, seed, scale, {}

    def logits(self, prefix):
        key = tuple(int(t) for t in prefix)
        if key not in self.memo:
            g = np.random.default_rng([self.seed, len(key)] + list(key))
            self.memo[key] = (g.normal(0, self.scale, self.V)).astype(np.float32)
        return self.memo[key]


def _round(target, drafter, ctx, nc, gamma, r):
    V = target.V
    drafts = np.zeros((nc, gamma), np.int32)
    zt = np.zeros((nc, gamma + 1, V), np.float32)
    zd = np.zeros((nc, gamma, V), np.float32)
    for c in range(nc):
        pre = list(ctx)
        for i in range(gamma):
            zd[c, i] = drafter.logits(pre)
            zt[c, i] = target.logits(pre)
            drafts[c, i] = r.choice(V, p=_softmax(zd[c, i]))
            pre.append(int(drafts[c, i]))
        zt[c, gamma] = target.logits(pre)
    u = r.random((nc, gamma + 1))
    n_acc, nxt, best, _ = recursive_accept(zt, zd, drafts, u)
    return [int(t) for t in drafts[best, : n_acc[best]]] + [int(nxt)]


@pytest.mark.parametrize("nc,gamma", [(2, 2), (3, 1), (4, 3)])
def test_monte_carlo_first_two_tokens(nc, gamma):
    V, n = 3, 12000
    target, drafter = _ToyModel(V, 11, 3.0), _ToyModel(V, 12, 1.0)
    r = np.random.default_rng(100 + nc)
    counts = np.zeros((V, V))
    for _ in range(n):
        out = []
        while len(out) < 2:
            out += _round(target, drafter, out, nc, gamma, r)
        counts[out[0], out[1]] += 1
    p1 = _softmax(target.logits([]))
    joint = np.array([[p1[a] * _softmax(target.logits([a]))[b] for b in range(V)] for a in range(V)])
    stat, pval = scipy.stats.chisquare(counts.ravel(), n * joint.ravel())
    assert pval > 1e-4, (counts, n * joint)


def test_q_equals_p_keeps_the_first_candidate():
    r = np.random.default_rng(3)
    nc, gamma, V = 4, 12, 512
    zt = r.normal(0, np.sqrt(2), (nc, gamma + 1, V)).astype(np.float32)
    zd = zt[:, :gamma].copy()
    for _ in range(10):
        drafts = r.integers(0, V, (nc, gamma)).astype(np.int32)
        n_acc, _, best, _ = recursive_accept(zt, zd, drafts, r.random((nc, gamma + 1)))
        assert int(best) == 0 and int(n_acc[0]) == gamma


def test_alive_bookkeeping_and_candidate_dispatch():
    """Candidates sharing the kept token stay alive; n_acc counts each one's drafts in the output."""
    V, gamma, nc = 5, 3, 3
    zt = np.zeros((1, nc, gamma + 1, V), np.float32)
    zd = np.zeros((1, nc, gamma, V), np.float32)          # uniform q; target uniform too: ratio 1, keep
    drafts = np.array([[[2, 1, 4], [2, 1, 0], [3, 3, 3]]], np.int32)
    u = np.full((1, nc, gamma + 1), 0.5)
    n_acc, nxt, best, marg = accept_candidates("recursive", zt, zd, drafts, u)
    assert list(n_acc[0]) == [3, 2, 0] and int(best[0]) == 0
    assert (nxt[0] == nxt[0, 0]).all()
