"""Oracle: lossless acceptance of a verified block (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Row i of the target logits (i = 0..gamma) is the target's prediction for the
token that follows block position i; draft t_m (m = 1..gamma) sits at block
position m.  Readings where the pages are silent:

* greedy ties resolve to the lowest token id; a bonus token is always emitted
  when every draft is accepted (no end-of-sequence in this setting);
* sampling: the ratio test is ``r * q(t) < p(t)`` (strict), inverse-CDF
  sampling walks token ids upward and takes the first cumulative sum strictly
  above ``r* x total`` (total = the last cumulative sum); the temperature
  divides both logit sets;
* uniforms[0..gamma-1] = r_1..r_gamma, uniforms[gamma] = r*.

Each decision's margin (distance from the threshold it was taken against,
relative to the threshold) is returned so that callers can tell decisions
that floating-point rounding could flip.
"""
from __future__ import annotations

import numpy as np


def _softmax(z: np.ndarray, temperature: float) -> np.ndarray:
    a = np.asarray(z, dtype=np.float64) / float(temperature)
    e = np.exp(a - a.max())
    return e / e.sum()


def _first_token_id(z: np.ndarray) -> tuple:
    """argmax with ties to the lowest id, and the gap to the runner-up."""
    z = np.asarray(z, dtype=np.float64)
    top = int(np.argmax(z))            # numpy returns the first maximal index
    rest = np.delete(z, top)
    gap = float(z[top] - rest.max()) if rest.size else float("inf")
    return top, gap


def greedy_accept(target_logits, drafts):
    """Greedy verification (ReaDy summary, section 3.1).

    The target accepts the longest draft prefix that matches its own argmax
    predictions; the first mismatch is replaced by the target's argmax (the
    correction), and if the whole block matches the target supplies a bonus
    token.  target_logits [P][V], drafts [gamma].  Returns (k, next, margin)
    where k is the number of accepted drafts and margin the smallest top-1 gap
    among the rows the decision read.
    """
    zt = np.asarray(target_logits)
    gamma = len(drafts)
    margin = float("inf")
    k = 0
    while True:
        g, gap = _first_token_id(zt[k])
        margin = min(margin, gap)
        if k == gamma or int(drafts[k]) != g:
            return k, g, margin
        k += 1


def _inverse_cdf(w: np.ndarray, r: float):
    """Smallest j whose running sum exceeds r * total (total = the full running sum).

    If rounding leaves no running sum above the threshold (r within an ulp of
    1), the last token with positive weight is taken.
    """
    csum = np.cumsum(w)
    total = float(csum[-1])
    target = r * total
    above = np.nonzero(csum > target)[0]
    j = int(above[0]) if above.size else int(np.nonzero(w > 0)[0][-1])
    margin = float(np.min(np.abs(csum - target))) / total
    return j, margin


def rejection_accept(target_logits, draft_logits, drafts, u, temperature: float = 1.0):
    """Speculative-sampling acceptance (ReaDy summary, section D.2; EvSpark Figure 1(c)).

    Drafts are checked left to right.  Draft t_i (drawn from q_i =
    softmax(draft_logits[i-1] / T)) is kept iff r_i * q_i(t_i) < p_{i-1}(t_i)
    with p_m = softmax(target_logits[m] / T); the remaining drafts are dropped
    at the first rejection.  After a rejection at i = k + 1 the correction is
    drawn from the residual max(0, p_k - q_{k+1}) (renormalised); after full
    acceptance the bonus is drawn from p_gamma.  Draws use r* by inverse CDF.
    This keeps the emitted tokens distributed as the target's.

    Returns (k, next_token, margin).
    """
    zt = np.asarray(target_logits)
    zd = np.asarray(draft_logits)
    gamma = len(drafts)
    margin = float("inf")
    k = gamma
    for i in range(1, gamma + 1):
        t = int(drafts[i - 1])
        p_prev = _softmax(zt[i - 1], temperature)
        q_i = _softmax(zd[i - 1], temperature)
        lhs = float(u[i - 1]) * q_i[t]
        rhs = p_prev[t]
        margin = min(margin, abs(lhs - rhs) / max(rhs, 1e-300))
        if not lhs < rhs:
            k = i - 1
            break
    p_k = _softmax(zt[k], temperature)
    if k < gamma:
        w = np.maximum(0.0, p_k - _softmax(zd[k], temperature))
        if not np.sum(w) > 0.0:          # cannot happen after a rejection; guard only
            w = p_k
    else:
        w = p_k
    nxt, m2 = _inverse_cdf(w, float(u[gamma]))
    return k, nxt, min(margin, m2)


def accept_candidates(mode, target_logits, draft_logits, drafts, u, temperature=1.0):
    """Acceptance for every candidate block of every sequence, then the winner.

    target_logits [nb][nc][P][V]; draft_logits [nb][nc][gamma][V] (sampling);
    drafts [nb][nc][gamma]; u [nb][nc][P] (sampling).  Each candidate is
    accepted on its own; the winner per sequence is the candidate with the
    most accepted drafts, the lowest index on ties (parity unpinned: the
    EvSpark digest reports multiple candidates but not the selection rule).
    Returns (n_acc [nb][nc], next [nb][nc], best [nb], margin [nb][nc]).
    """
    zt = np.asarray(target_logits)
    nb, nc = zt.shape[:2]
    n_acc = np.zeros((nb, nc), np.int32)
    nxt = np.zeros((nb, nc), np.int32)
    marg = np.zeros((nb, nc))
    best = np.zeros(nb, np.int32)
    for b in range(nb):
        for c in range(nc):
            if mode == "greedy":
                k, t, m = greedy_accept(zt[b, c], drafts[b, c])
            else:
                k, t, m = rejection_accept(zt[b, c], draft_logits[b, c], drafts[b, c], u[b, c], temperature)
            n_acc[b, c], nxt[b, c], marg[b, c] = k, t, m
        best[b] = int(np.argmax(n_acc[b]))
    return n_acc, nxt, best, marg
