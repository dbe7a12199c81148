"""Oracle: verification of a token tree in one block forward, its acceptance and its slice (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The EvSpark digest reports several candidate blocks per decoding step
(Interpretation: C = 1/2/4) and the ReaDy summary lists tree verification with
recovery of recurrent state as related work (section 5); neither prints a rule
or an equation.  Plain reading used here:

* A tree of n nodes per sequence: node 0 is the anchor, every other node m has
  a parent p(m) < m and carries a drafted token.  Node m stands for the token
  sequence along the path root -> m; candidate blocks that share a prefix share
  the nodes of that prefix, which are then computed once.
* Forward: every output at node m equals what a chain block forward over the
  path root -> m (``verify_block``) gives at its last position.  Written out:
  the FIR windows of node m read its ancestors, newest first, and then the
  committed window; its IIR state starts from its parent's state (the
  committed state for the root); its query attends to the committed prefix and
  to the block keys of its ancestors and itself (the tree mask).
* Greedy acceptance walks from the root: at node m the target's argmax
  (ties to the lowest id) is compared with m's children in index order; the
  first child holding it becomes the current node; otherwise the argmax is
  emitted.  With a chain this is the ReaDy summary's section 3.1 rule.
* Sampling acceptance applies the section D.2 ratio test to the children of the
  current node in index order against a running residual (multi-step
  speculative sampling with one draft distribution per child): child c with
  token t drawn from q_c = softmax(draft row c / T) is kept iff
  r_c * q_c(t) * z < w(t), where w / z is the current residual of the target
  row p (w = p, z = 1 at each node); a rejection sets w <- max(0, w - z q_c),
  z <- sum(w).  A kept child becomes the current node; if every child is
  rejected the next token is drawn from w, and at a node without children the
  bonus is drawn from p.  Draws use r* by inverse CDF.  When each child's token
  is an independent draw from its q_c, every emitted token is distributed as
  the target's.  With a chain this is exactly ``rejection_accept``.
* Slicing commits the accepted path: the positions of the path play the role
  of block rows 0..k of ``slice_state``.

Uniforms: u[m] for m >= 1 is node m's test uniform; u[0] (the anchor has no
test) is r*.
"""
from __future__ import annotations

import math
from typing import List

import numpy as np

from .acceptance import _first_token_id, _inverse_cdf, _residual, _softmax
from .layer import Layer, SeqState, as_f64
from .slicing import slice_state


def check_tree(parent) -> np.ndarray:
    """The parent array as int64, after checking parent[0] = -1 and 0 <= parent[m] < m."""
    par = np.asarray(parent, dtype=np.int64)
    assert par.ndim == 1 and par.size >= 1 and par[0] == -1, "node 0 is the anchor (parent -1)"
    for m in range(1, par.size):
        assert 0 <= par[m] < m, f"node {m}: parent {par[m]} must precede it"
    return par


def tree_path(parent, m: int) -> List[int]:
    """Nodes root -> m."""
    par = check_tree(parent)
    path = [int(m)]
    while path[-1] != 0:
        path.append(int(par[path[-1]]))
    return path[::-1]


def children(parent, m: int) -> List[int]:
    """Children of node m in index order."""
    par = check_tree(parent)
    return [c for c in range(par.size) if par[c] == m]


def _lagged(rows: np.ndarray, window: np.ndarray, par: np.ndarray, m: int, j: int) -> np.ndarray:
    """The input j positions before node m along its path: an ancestor's row (j <= depth of m), else
    a row of the committed window (oldest first: lag depth + 1 is its last row)."""
    cur, steps = m, 0
    while steps < j and cur > 0:
        cur = int(par[cur])
        steps += 1
    if steps == j:
        return rows[cur]
    back = j - steps                     # the anchor was reached; 1 = the newest committed input
    return window[window.shape[0] - back]


def tree_fir(rows, window, taps, parent) -> np.ndarray:
    """Depthwise FIR at every node over its own history: out_m = sum_j taps[j] * in(m, j),
    in(m, j) = the input j positions before m along its path (ancestors, then the window)."""
    par = check_tree(parent)
    r = as_f64(rows)
    win = as_f64(window)
    w = as_f64(taps)
    n, d = r.shape
    assert win.shape[0] == w.shape[0] - 1
    out = np.zeros((n, d))
    for m in range(n):
        acc = np.zeros(d)
        for j in range(w.shape[0]):
            acc = acc + w[j] * _lagged(r, win, par, m, j)
        out[m] = acc
    return out


def tree_iir(g, s_prev, lam, beta, c, parent):
    """Modal IIR along the tree: s_m = lam * s_{p(m)} + beta * g_m (s of the anchor's parent =
    the committed state), y_m = sum_n c * s_m.  Returns (s [n][d][N], y [n][d])."""
    par = check_tree(parent)
    gg = as_f64(g)
    lam, beta, c = as_f64(lam), as_f64(beta), as_f64(c)
    s0 = as_f64(s_prev)
    n, d = gg.shape
    S = np.zeros((n,) + s0.shape)
    Y = np.zeros((n, d))
    for m in range(n):
        prev = s0 if m == 0 else S[par[m]]
        S[m] = lam * prev + beta * gg[m][:, None]
        Y[m] = (c * S[m]).sum(axis=1)
    return S, Y


def tree_attention(q, k_blk, v_blk, k_blocks, v_blocks, parent) -> np.ndarray:
    """Every node's query against the committed keys and the block keys of its ancestors and
    itself; explicit score matrix over all block keys with the others set to -inf."""
    par = check_tree(parent)
    qq, kb, vb = as_f64(q), as_f64(k_blk), as_f64(v_blk)
    n, H, Dh = qq.shape
    visible = np.zeros((n, n), bool)               # visible[m, j]: block key j is on m's path
    for m in range(n):
        a = m
        while True:
            visible[m, a] = True
            if a == 0:
                break
            a = int(par[a])
    o = np.zeros((n, H, Dh))
    scale = 1.0 / math.sqrt(Dh)
    for h in range(H):
        pre_k = [as_f64(b[h]) for b in k_blocks]
        pre_v = [as_f64(b[h]) for b in v_blocks]
        keys = np.concatenate(pre_k + [kb[:, h, :]], axis=0)
        vals = np.concatenate(pre_v + [vb[:, h, :]], axis=0)
        L = keys.shape[0] - n
        for m in range(n):
            sc = keys @ qq[m, h] * scale
            sc[L:][~visible[m]] = -np.inf
            w = np.exp(sc - sc.max())
            o[m, h] = (w / w.sum()) @ vals
    return o


def tree_verify(layer: Layer, st: SeqState, parent, x, q, k, v):
    """One block forward over every node of the tree from the committed state (only read).

    x [n][d], q/k/v [n][H][Dh].  Returns dict f [n][d], s [n][d][N], y [n][d], o [n][H][Dh]."""
    f = tree_fir(x, st.short_win, layer.w_short, parent)
    g = tree_fir(f, st.outer_win, layer.w_outer, parent)
    s, y = tree_iir(g, st.iir, layer.lam, layer.beta, layer.c, parent)
    o = tree_attention(q, k, v, st.k_blocks, st.v_blocks, parent)
    return {"f": f, "s": s, "y": y, "o": o}


def tree_greedy_accept(target_logits, parent, tokens):
    """Greedy walk from the anchor.  target_logits [n][V] (row m predicts the token after node m),
    tokens [n] (tokens[0] unused).  Returns (k, path, next, margin): k = depth of the accepted
    node, path = its nodes root -> node, margin = smallest top-1 gap of the rows read."""
    par = check_tree(parent)
    zt = np.asarray(target_logits)
    m, path, margin = 0, [0], float("inf")
    while True:
        g, gap = _first_token_id(zt[m])
        margin = min(margin, gap)
        nxt = [c for c in children(par, m) if int(tokens[c]) == g]
        if not nxt:
            return len(path) - 1, path, g, margin
        m = nxt[0]
        path.append(m)


def tree_rejection_accept(target_logits, draft_logits, parent, tokens, u, temperature: float = 1.0):
    """Sampling walk from the anchor (multi-step speculative sampling over each node's children).

    target_logits [n][V]; draft_logits [n][V]: row c is the distribution node c's token was drawn
    from (row 0 unused); tokens [n]; u [n]: u[c] is node c's test uniform, u[0] = r*.  Returns
    (k, path, next, margin) as ``tree_greedy_accept``, margin = smallest relative distance of a
    ratio test or of the final draw from its threshold."""
    par = check_tree(parent)
    zt, zd = np.asarray(target_logits), np.asarray(draft_logits)
    V = zt.shape[1]
    m, path, margin = 0, [0], float("inf")
    while True:
        w = _softmax(zt[m], temperature)
        z = 1.0
        kept = None
        for c in children(par, m):
            t = int(tokens[c])
            q = _softmax(zd[c], temperature)
            if 0 <= t < V:
                lhs = float(u[c]) * q[t] * z
                rhs = w[t]
                margin = min(margin, abs(lhs - rhs) / max(rhs, 1e-300))
                if lhs < rhs:
                    kept = c
                    break
            w, z = _residual(w, z, q)
        if kept is None:
            nxt, m2 = _inverse_cdf(w, float(u[0]))
            return len(path) - 1, path, nxt, min(margin, m2)
        m = kept
        path.append(m)


def tree_slice(st: SeqState, x, fwd, k_blk, v_blk, path) -> SeqState:
    """Commit the accepted path: its nodes, in order, are the block rows 0..k of ``slice_state``."""
    idx = np.asarray(path, dtype=np.int64)
    chain_fwd = {"f": np.asarray(fwd["f"])[idx], "s": np.asarray(fwd["s"])[idx]}
    return slice_state(st, np.asarray(x)[idx], chain_fwd, np.asarray(k_blk)[idx], np.asarray(v_blk)[idx],
                       len(path) - 1)
