"""Pins for the oracle's token-tree verification, acceptance and slicing (CPU only).

* every node's forward equals the chain forward over its root-to-node path
  (``verify_block``, itself pinned by closed forms and brute force), on chains,
  stars, random trees and trees deeper than the outer FIR window;
* the tree mask: a node's attention output ignores every non-ancestor's keys and
  values and changes with an ancestor's;
* a planted mistake (parents read as the previous node) breaks the identity;
* greedy: a chain is the one-block rule; on random trees the accepted node is
  the deepest node whose every edge follows the parent's argmax (brute force);
* sampling: a chain is the one-block rejection rule bit for bit; the first
  emitted token is distributed exactly as the target's over every combination
  of children tokens (decision boundaries by bisection), with each child
  drawn from its own draft distribution; planted mistakes in the residual break
  that identity; Monte Carlo: the first two emitted tokens follow the target's
  joint law under a prefix-keyed toy target and drafter with depth-2 trees;
* slicing: tree forward + slice along the accepted path = sequential
  single-position steps over the path (the replay definition).
"""
import itertools

import numpy as np
import pytest
import scipy.stats

import oracle
import oracle.tree as tree_mod
from oracle.tree import (children, tree_greedy_accept, tree_path, tree_rejection_accept, tree_slice,
                         tree_verify)

EPS1 = 1.0 - 1e-16


def _softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def _layer_state(rng, d=6, Ts=3, To=7, N=4, H=2, Dh=8, L=9):
    lay = oracle.Layer(rng.normal(0, Ts ** -0.5, (Ts, d)), rng.normal(0, To ** -0.5, (To, d)),
                       rng.uniform(0.5, 0.99, (d, N)), rng.normal(0, 0.25, (d, N)), rng.normal(0, 0.25, (d, N)))
    st = oracle.SeqState(rng.normal(0, 1, (Ts - 1, d)), rng.normal(0, 1, (To - 1, d)), rng.normal(0, 0.5, (d, N)),
                         [rng.normal(0, 1, (H, L, Dh))], [rng.normal(0, 1, (H, L, Dh))])
    return lay, st


def _tree(kind, n, rng):
    if kind == "chain":
        return np.array([-1] + list(range(n - 1)))
    if kind == "star":
        return np.array([-1] + [0] * (n - 1))
    par = [-1]
    for m in range(1, n):
        par.append(int(rng.integers(0, m)))
    return np.array(par)


def _inputs(rng, n, d, H, Dh):
    return (rng.normal(0, 1, (n, d)), rng.normal(0, 1, (n, H, Dh)), rng.normal(0, 1, (n, H, Dh)),
            rng.normal(0, 1, (n, H, Dh)))


@pytest.mark.parametrize("kind,n,To", [("chain", 7, 7), ("star", 6, 7), ("random", 9, 7), ("random", 12, 4),
                                       ("random", 1, 7), ("chain", 10, 3), ("random", 16, 16)])
def test_every_node_equals_its_chain_forward(kind, n, To):
    rng = np.random.default_rng(n * 31 + To)
    lay, st = _layer_state(rng, To=To)
    par = _tree(kind, n, rng)
    x, q, k, v = _inputs(rng, n, 6, 2, 8)
    fwd = tree_verify(lay, st, par, x, q, k, v)
    for m in range(n):
        p = tree_path(par, m)
        ref = oracle.verify_block(lay, st, x[p], q[p], k[p], v[p])
        for key in ("f", "s", "y", "o"):
            np.testing.assert_allclose(fwd[key][m], ref[key][-1], rtol=1e-12, atol=1e-12, err_msg=f"{key}[{m}]")


def test_chain_tree_is_the_block_forward():
    rng = np.random.default_rng(3)
    lay, st = _layer_state(rng)
    n = 8
    x, q, k, v = _inputs(rng, n, 6, 2, 8)
    fwd = tree_verify(lay, st, _tree("chain", n, rng), x, q, k, v)
    ref = oracle.verify_block(lay, st, x, q, k, v)
    for key in ("f", "s", "y", "o"):
        np.testing.assert_allclose(fwd[key], ref[key], rtol=1e-12, atol=1e-12)


def test_planted_previous_node_mistake_is_caught():
    """Reading node m - 1 as the parent (the chain layout) is wrong on a branching tree."""
    rng = np.random.default_rng(4)
    lay, st = _layer_state(rng)
    par = np.array([-1, 0, 0, 1, 2, 2])
    x, q, k, v = _inputs(rng, len(par), 6, 2, 8)
    wrong = tree_verify(lay, st, _tree("chain", len(par), rng), x, q, k, v)
    bad = 0
    for m in range(len(par)):
        p = tree_path(par, m)
        ref = oracle.verify_block(lay, st, x[p], q[p], k[p], v[p])
        bad += not np.allclose(wrong["y"][m], ref["y"][-1]) or not np.allclose(wrong["o"][m], ref["o"][-1])
    assert bad >= 3


def test_tree_mask_ignores_non_ancestors():
    rng = np.random.default_rng(5)
    lay, st = _layer_state(rng)
    par = np.array([-1, 0, 0, 1, 1, 2, 3])
    x, q, k, v = _inputs(rng, len(par), 6, 2, 8)
    base = tree_verify(lay, st, par, x, q, k, v)
    m = 6                                                   # path 0 -> 1 -> 3 -> 6
    anc = set(tree_path(par, m))
    for j in range(len(par)):
        k2, v2, x2 = k.copy(), v.copy(), x.copy()
        k2[j] += 3.0
        v2[j] -= 2.0
        x2[j] += 1.5
        out = tree_verify(lay, st, par, x2, q, k2, v2)
        same_o = np.array_equal(out["o"][m], base["o"][m])
        same_y = np.array_equal(out["y"][m], base["y"][m])
        assert same_o == (j not in anc) and same_y == (j not in anc), j


@pytest.mark.parametrize("gamma,V", [(0, 7), (1, 3), (6, 40), (12, 512)])
def test_greedy_chain_is_the_block_rule(gamma, V):
    rng = np.random.default_rng(gamma + V)
    for trial in range(20):
        zt = rng.normal(0, np.sqrt(2), (gamma + 1, V)).astype(np.float32)
        drafts = np.argmax(zt[:gamma], axis=1).astype(np.int32)
        if gamma and trial % 2:
            drafts[rng.integers(0, gamma)] = rng.integers(0, V)
        tokens = np.concatenate([[0], drafts])
        k, path, nxt, marg = tree_greedy_accept(zt, _tree("chain", gamma + 1, rng), tokens)
        assert (k, nxt, marg) == oracle.greedy_accept(zt, drafts)
        assert path == list(range(k + 1))


def test_greedy_random_trees_brute_force():
    """The accepted node is the deepest one whose every edge (a -> b) has b holding the argmax of
    a's row and no earlier sibling of b holding it."""
    rng = np.random.default_rng(6)
    for trial in range(200):
        n, V = int(rng.integers(1, 14)), int(rng.integers(2, 5))
        par = _tree("random", n, rng)
        zt = rng.normal(0, 1, (n, V))
        tokens = rng.integers(0, V, n)
        top = np.argmax(zt, axis=1)

        def consistent(m):
            p = tree_path(par, m)
            for a, b in zip(p[:-1], p[1:]):
                first = [c for c in range(n) if par[c] == a and tokens[c] == top[a]]
                if not first or first[0] != b:
                    return False
            return True

        best = max((m for m in range(n) if consistent(m)), key=lambda m: len(tree_path(par, m)))
        k, path, nxt, _ = tree_greedy_accept(zt, par, tokens)
        assert path == tree_path(par, best) and k == len(path) - 1 and nxt == int(top[best])


@pytest.mark.parametrize("gamma,V,T", [(0, 7, 1.0), (1, 3, 1.0), (6, 512, 0.5), (12, 512, 2.0)])
def test_sampling_chain_is_the_rejection_rule(gamma, V, T):
    rng = np.random.default_rng(gamma * 7 + V)
    for trial in range(30):
        zt = rng.normal(0, np.sqrt(2), (gamma + 1, V)).astype(np.float32)
        zd = rng.normal(0, np.sqrt(2), (gamma, V)).astype(np.float32)
        if trial % 3 == 0 and gamma:
            zd[: gamma // 2] = zt[: gamma // 2]
        drafts = np.array([rng.choice(V, p=_softmax(zd[i] / T)) for i in range(gamma)], np.int32)
        u = rng.random(gamma + 1)
        tokens = np.concatenate([[0], drafts])
        zd_tree = np.concatenate([np.zeros((1, V), np.float32), zd])       # row c: node c's distribution
        u_tree = np.concatenate([[u[gamma]], u[:gamma]])                    # u[0] = r*
        k, path, nxt, marg = tree_rejection_accept(zt, zd_tree, _tree("chain", gamma + 1, rng), tokens, u_tree, T)
        assert (k, nxt, marg) == oracle.rejection_accept(zt, zd, drafts, u, T)
        assert path == list(range(k + 1))


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
    if not f(0.0):
        return 0.0
    if f(EPS1):
        return 1.0
    return _boundary(f, 0.0, EPS1)


def _draw_measure(tok, dist, weight):
    cur, left = 0.0, 0.0
    while tok(cur) != tok(EPS1):
        edge = _boundary(tok, cur, EPS1)
        dist[tok(cur)] += weight * (edge - left)
        left = edge
        cur = edge + 1e-15
    dist[tok(EPS1)] += weight * (1.0 - left)


def _exact_first_token(zt, zd, par, V, accept=tree_rejection_accept):
    """P(first emitted token = y) for a root with children 1..m (each child's token an independent
    draw from its own row of zd), summed over every combination of children tokens."""
    kids = children(par, 0)
    qs = {c: _softmax(zd[c]) for c in kids}
    dist = np.zeros(V)
    for combo in itertools.product(range(V), repeat=len(kids)):
        tokens = np.zeros(len(par), np.int64)
        for c, t in zip(kids, combo):
            tokens[c] = t
        prob = float(np.prod([qs[c][t] for c, t in zip(kids, combo)]))
        reach = 1.0
        for i, c in enumerate(kids):
            def kept(r, i=i, c=c):
                u = np.full(len(par), 0.5)
                for c2 in kids[:i]:
                    u[c2] = EPS1
                u[c] = r
                k, path, _, _ = accept(zt, zd, par, tokens, u)
                return k >= 1 and path[1] == c
            a = _accept_fraction(kept)
            dist[combo[i]] += prob * reach * a
            reach *= 1.0 - a
            if reach == 0.0:
                break
        if reach > 0.0:
            def tok(rs):
                u = np.full(len(par), EPS1)
                u[0] = rs
                return int(accept(zt, zd, par, tokens, u)[2])
            _draw_measure(tok, dist, prob * reach)
    return dist


@pytest.mark.parametrize("m,V,seed", [(1, 3, 0), (2, 3, 1), (2, 4, 2), (3, 3, 3)])
def test_first_token_is_target_distributed_exactly(m, V, seed):
    rng = np.random.default_rng(seed)
    par = np.array([-1] + [0] * m)
    zt = rng.normal(0, np.sqrt(2), (m + 1, V))
    zd = rng.normal(0, np.sqrt(2), (m + 1, V))          # a different draft distribution per child
    dist = _exact_first_token(zt, zd, par, V)
    np.testing.assert_allclose(dist, _softmax(zt[0]), atol=1e-9)


@pytest.mark.parametrize("plant", ["no_update", "first_child_q"])
def test_planted_residual_mistakes_break_the_law(plant, monkeypatch):
    rng = np.random.default_rng(0)          # after child 1's rejection the residual keeps 3 of 4 tokens
    par = np.array([-1, 0, 0])
    zt = rng.normal(0, np.sqrt(2), (3, 4))
    zd = rng.normal(0, np.sqrt(2), (3, 4))
    if plant == "no_update":
        monkeypatch.setattr(tree_mod, "_residual", lambda w, z, q: (w, z))
        accept = tree_rejection_accept
    else:
        def accept(zt_, zd_, par_, tokens, u, T=1.0):
            zd2 = zd_.copy()
            zd2[2] = zd_[1]                                  # test child 2 against child 1's distribution
            return tree_rejection_accept(zt_, zd2, par_, tokens, u, T)
    dist = _exact_first_token(zt, zd, par, 4, accept)
    assert np.max(np.abs(dist - _softmax(zt[0]))) > 1e-3


def test_two_emitted_tokens_follow_the_joint_law():
    """Depth-2 trees (root -> 2 children -> 2 children each), tokens drawn from a prefix-keyed toy
    drafter; a round that emits one token is followed by a round from the new prefix (a root-only
    tree, whose bonus is drawn from the target).  The first two emitted tokens follow p(a) p(b|a)."""
    V = 3
    g = np.random.default_rng(11)
    tgt = {(): g.normal(0, 1.2, V)}
    drf = {(): g.normal(0, 1.2, V)}
    for a in range(V):
        tgt[(a,)] = g.normal(0, 1.2, V)
        drf[(a,)] = g.normal(0, 1.2, V)
        for b in range(V):
            tgt[(a, b)] = g.normal(0, 1.2, V)
    par = np.array([-1, 0, 0, 1, 1, 2, 2])
    rng = np.random.default_rng(12)
    counts = np.zeros((V, V))
    trials = 40000
    for _ in range(trials):
        tokens = np.zeros(7, np.int64)
        for c in (1, 2):
            tokens[c] = rng.choice(V, p=_softmax(drf[()]))
        for c in (3, 4, 5, 6):
            tokens[c] = rng.choice(V, p=_softmax(drf[(int(tokens[par[c]]),)]))
        prefix = {0: ()}
        for c in range(1, 7):
            prefix[c] = prefix[par[c]] + (int(tokens[c]),)
        zt = np.stack([tgt[prefix[c]] for c in range(7)])
        zd = np.stack([np.zeros(V)] + [drf[prefix[par[c]]] for c in range(1, 7)])
        k, path, nxt, _ = tree_rejection_accept(zt, zd, par, tokens, rng.random(7))
        emitted = [int(tokens[c]) for c in path[1:]] + [nxt]
        if len(emitted) < 2:
            emitted.append(int(rng.choice(V, p=_softmax(tgt[tuple(emitted)]))))
        counts[emitted[0], emitted[1]] += 1
    p1 = _softmax(tgt[()])
    expect = np.array([[p1[a] * _softmax(tgt[(a,)])[b] for b in range(V)] for a in range(V)]) * trials
    chi2, pval = scipy.stats.chisquare(counts.ravel(), expect.ravel())
    assert pval > 1e-3, (chi2, pval)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_slice_equals_sequential_steps_over_the_path(seed):
    rng = np.random.default_rng(seed)
    lay, st = _layer_state(rng, To=5)
    n = 10
    par = _tree("random", n, rng)
    x, q, k, v = _inputs(rng, n, 6, 2, 8)
    fwd = tree_verify(lay, st, par, x, q, k, v)
    for m in range(n):
        path = tree_path(par, m)
        new = tree_slice(st, x, fwd, k, v, path)
        ref, _ = oracle.sequential_steps(lay, st, x[path], q[path], k[path], v[path], len(path))
        np.testing.assert_allclose(new.short_win, ref.short_win, rtol=0, atol=0)
        np.testing.assert_allclose(new.outer_win, ref.outer_win, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(new.iir, ref.iir, rtol=1e-12, atol=1e-12)
        assert new.kv_len == ref.kv_len == st.kv_len + len(path)
        np.testing.assert_array_equal(np.concatenate(new.k_blocks, axis=1), np.concatenate(ref.k_blocks, axis=1))
