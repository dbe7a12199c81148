"""Pins for the oracle's drafter (CPU only).

* serial sampling: the first draft's law is softmax((z_0 + B[anchor]) / T) and
  the second's, given the first, softmax((z_1 + B[t_1]) / T), measured
  exactly by locating the sampler's own decision boundaries (bisection);
* the trunk is causal over the block rows (a shorter block gives the same
  leading logits) and every window row reaches the logits;
The architecture is a reading (the pages print no equations): parity
unpinned beyond these.
"""
import numpy as np
import pytest

from oracle import drafter as OD

EPS1 = 1.0 - 1e-16


def _softmax(z):
    z = np.asarray(z, np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def _boundary(f, lo, hi, iters=80):
    flo = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) == flo:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _law(tok, V):
    """Measure of u in [0, 1) mapped to each token by a monotone step function tok(u)."""
    dist = np.zeros(V)
    cur, left = 0.0, 0.0
    while tok(cur) != tok(EPS1):
        edge = _boundary(tok, cur, EPS1)
        dist[tok(cur)] += edge - left
        left, cur = edge, edge + 1e-15
    dist[tok(EPS1)] += 1.0 - left
    return dist


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_first_and_second_draft_laws(T):
    r = np.random.default_rng(3)
    V, gamma, anchor = 5, 2, 3
    z = r.normal(0, 1.5, (gamma, V)).astype(np.float32)
    B = r.normal(0, 1.5, (V, V)).astype(np.float32)
    q1 = _softmax((z[0] + B[anchor]).astype(np.float64) / T)          # the bias is added in fp32
    law1 = _law(lambda u: int(OD.draft_sample(z, B, anchor, [u, 0.5], T)[0][0]), V)
    np.testing.assert_allclose(law1, q1, atol=1e-9)
    for first in range(V):
        u1 = sum(q1[:first]) + 0.5 * q1[first]                        # inside the interval that draws `first`
        assert int(OD.draft_sample(z, B, anchor, [u1, 0.5], T)[0][0]) == first
        law2 = _law(lambda u: int(OD.draft_sample(z, B, anchor, [u1, u], T)[0][1]), V)
        np.testing.assert_allclose(law2, _softmax((z[1] + B[first]).astype(np.float64) / T), atol=1e-9)


def _tiny(r, d=16, H=2, V=11, dt=24, F=32):
    layers = [OD.TrunkLayer(g1=1 + 0.1 * r.standard_normal(d), w_qkv=r.standard_normal((d, 3 * d)) / np.sqrt(d),
                            w_o=r.standard_normal((d, d)) / np.sqrt(d), g2=1 + 0.1 * r.standard_normal(d),
                            w_up=r.standard_normal((d, F)) / np.sqrt(d), w_down=r.standard_normal((F, d)) / np.sqrt(F))
              for _ in range(2)]
    return OD.Drafter(w_proj=r.standard_normal((dt, d)) / np.sqrt(dt), emb=r.standard_normal((V, d)),
                      mask=r.standard_normal(d), markov=r.standard_normal((V, V)).astype(np.float32), layers=layers,
                      g_f=np.ones(d), heads=H, eps=1e-6)


def test_trunk_is_causal_and_reads_the_whole_window():
    r = np.random.default_rng(4)
    dr = _tiny(r)
    win = r.standard_normal((9, 24))
    z12 = OD.draft_logits(dr, win, 5, 12, rounding=False)
    z4 = OD.draft_logits(dr, win, 5, 4, rounding=False)
    np.testing.assert_allclose(z12[:4], z4, atol=1e-12)                  # later rows never reach earlier ones
    for j in (0, 8):                                                      # the oldest and the newest window row
        w2 = win.copy()
        w2[j] += 1.0
        assert np.abs(OD.draft_logits(dr, w2, 5, 4, rounding=False)[0] - z4[0]).max() > 1e-6
    z_other = OD.draft_logits(dr, win, 6, 4, rounding=False)             # the anchor reaches every row
    assert (np.abs(z_other - z4).max(axis=1) > 1e-6).all()
