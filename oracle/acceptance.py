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


def _residual(w: np.ndarray, z: float, q: np.ndarray):
    """One rejection: the next residual weights max(0, w - z q) and their total.

    w holds unnormalised weights whose normalised form w / z is the current
    target distribution; the result keeps the same convention.  If rounding
    leaves no positive weight (a rejection implies some token has more
    target than draft mass, so this cannot happen in exact arithmetic) the
    weights stay as they were.
    """
    w2 = np.maximum(0.0, w - z * q)
    z2 = float(np.sum(w2))
    if not z2 > 0.0:
        return w, z
    return w2, z2


def recursive_accept(target_logits, draft_logits, drafts, u, temperature: float = 1.0):
    """Lossless acceptance over several candidate blocks of one sequence.

    A multi-draft generalisation of the ReaDy summary's section D.2 rule for
    the C = 1/2/4 candidate blocks of the EvSpark digest (Interpretation);
    the pages state no rule for several candidates, so this follows the
    published recursive rejection scheme for multiple drafts (SpecInfer's
    multi-step speculative sampling).  All candidates share the anchor; at
    depth k the alive candidates are those whose drafts t_1..t_k equal the
    accepted prefix, and the lowest-index alive candidate supplies the rows
    p = softmax(target row k / T) and q = softmax(draft row k / T) (rows of
    candidates that share a prefix are the same distributions).  Alive
    candidates are tried in index order: draft t is kept iff
    r * q(t) < w(t) / z for the current residual w / z (w = p, z = 1 at the
    start of a depth); a rejection replaces w by max(0, w - z q).  The first
    kept draft extends the prefix and the candidates holding it stay alive;
    if every alive candidate is rejected the next token is drawn from the
    final residual, and after gamma kept drafts the bonus is drawn from
    p_gamma.  Draws use r* = u[0][gamma] by inverse CDF.  When the drafts of
    the alive candidates are independent draws from q, every emitted token
    is distributed as the target's.  With one candidate this is exactly
    ``rejection_accept``.

    target_logits [nc][P][V]; draft_logits [nc][gamma][V]; drafts [nc][gamma];
    u [nc][P]: candidate c's depth-k test uses u[c][k].  Returns (n_acc [nc],
    next, best, margin [nc]): n_acc[c] counts candidate c's leading drafts
    that are in the accepted sequence, best is the lowest-index candidate
    alive at the end (n_acc[best] = k), margin[c] is the smallest relative
    distance of candidate c's tests from their thresholds (the final draw's
    margin goes to best).
    """
    zt = np.asarray(target_logits)
    zd = np.asarray(draft_logits)
    dr = np.asarray(drafts)
    nc, P, V = zt.shape
    gamma = P - 1
    margin = np.full(nc, np.inf)
    n_acc = np.zeros(nc, np.int32)
    alive = list(range(nc))
    k = 0
    while True:
        rep = alive[0]
        w = _softmax(zt[rep, k], temperature)
        if k == gamma:                        # every draft of the alive path kept: bonus from p_gamma
            break
        z = 1.0
        q = _softmax(zd[rep, k], temperature)
        kept = None
        for c in alive:
            t = int(dr[c, k])
            if 0 <= t < V:
                lhs = float(u[c, k]) * q[t] * z
                rhs = w[t]
                margin[c] = min(margin[c], abs(lhs - rhs) / max(rhs, 1e-300))
                if lhs < rhs:
                    kept = t
                    break
            w, z = _residual(w, z, q)
        if kept is None:
            break
        for c in alive:
            if int(dr[c, k]) != kept:
                n_acc[c] = k
        alive = [c for c in alive if int(dr[c, k]) == kept]
        k += 1
    for c in alive:
        n_acc[c] = k
    best = alive[0]
    nxt, m2 = _inverse_cdf(w, float(u[0, gamma]))
    margin[best] = min(margin[best], m2)
    return n_acc, nxt, best, margin


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
        if mode == "recursive":
            n_acc[b], t, best[b], marg[b] = recursive_accept(zt[b], draft_logits[b], drafts[b], u[b], temperature)
            nxt[b] = t
            continue
        for c in range(nc):
            if mode == "greedy":
                k, t, m = greedy_accept(zt[b, c], drafts[b, c])
            else:
                k, t, m = rejection_accept(zt[b, c], draft_logits[b, c], drafts[b, c], u[b, c], temperature)
            n_acc[b, c], nxt[b, c], marg[b, c] = k, t, m
        best[b] = int(np.argmax(n_acc[b]))
    return n_acc, nxt, best, marg
