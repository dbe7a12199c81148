"""Oracle: one initial-state block forward of the synthetic hybrid layer (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer holds the three state classes the EvSpark digest names
(Synopsis; Interpretation: "finite convolution windows, modal IIR states,
and attention caches"):

  conv/recurrent path   x -> short depthwise FIR -> f -> outer depthwise FIR
                        -> g -> diagonal modal IIR -> y
  attention path        (q, k, v) -> causal block attention over the KV prefix -> o

Figure 1(d) of the digest names the outer-FIR inputs u and the IIR states s_i;
here f_i is that u_i.  The pages give no equations; the plain readings used:

* FIR taps multiply lags (convolution): out_i = sum_j w[j] * in[i - j], where
  negative indices read the committed window (oldest first, newest last).
* IIR: s_i = lam * s_{i-1} + beta * g_i (per channel, per pole, lam given
  directly, no discretisation); y_i = sum_n c * s_i (state after the update).
* attention: query i sees every committed key and block keys 0..i,
  score = q . k / sqrt(Dh), softmax, weighted sum of values; no positional
  encoding, one KV head per query head.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np


def as_f64(a) -> np.ndarray:
    """Exact float64 copy of an fp32/fp64 array or of uint16 bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@dataclasses.dataclass
class Layer:
    """Fixed per-layer parameters (fp32 arrays, widened to fp64 when used)."""
    w_short: np.ndarray   # [Ts][d]
    w_outer: np.ndarray   # [To][d]
    lam: np.ndarray       # [d][N]
    beta: np.ndarray      # [d][N]
    c: np.ndarray         # [d][N]

    @classmethod
    def from_dict(cls, p) -> "Layer":
        return cls(p["w_short"], p["w_outer"], p["lam"], p["beta"], p["c"])


@dataclasses.dataclass
class SeqState:
    """Committed state of one sequence.

    short_win [Ts-1][d] and outer_win [To-1][d] hold the last inputs of the two
    FIRs, oldest first; iir [d][N]; the KV cache is a list of row blocks, each
    [H][n][Dh] (any dtype accepted by ``as_f64``), whose concatenation along
    the row axis is the readable prefix.
    """
    short_win: np.ndarray
    outer_win: np.ndarray
    iir: np.ndarray
    k_blocks: List[np.ndarray]
    v_blocks: List[np.ndarray]

    @property
    def kv_len(self) -> int:
        return int(sum(b.shape[1] for b in self.k_blocks))

    def copy(self) -> "SeqState":
        return SeqState(self.short_win.copy(), self.outer_win.copy(), self.iir.copy(),
                        list(self.k_blocks), list(self.v_blocks))


def depthwise_fir(block: np.ndarray, window: np.ndarray, taps: np.ndarray) -> np.ndarray:
    """Causal depthwise FIR of a block of P positions against a committed window.

    block [P][d], window [W][d] (W = taps-1 inputs before the block, oldest
    first), taps [T][d].  out_i[ch] = sum_{j<T} taps[j][ch] * in[i-j][ch], with
    in[m] = block[m] for m >= 0 and window[W + m] for m < 0.  Used for both the
    short FIR (x -> f) and the outer FIR (f -> g): the finite convolution
    windows of the EvSpark digest (Interpretation; Figure 1(d)).
    """
    blk = as_f64(block)
    win = as_f64(window)
    w = as_f64(taps)
    P, d = blk.shape
    T = w.shape[0]
    W = win.shape[0]
    assert W == T - 1, "window must hold taps-1 inputs"
    full = np.concatenate([win, blk], axis=0)       # index m of the text is row W + m
    out = np.zeros((P, d))
    for i in range(P):
        acc = np.zeros(d)
        for j in range(T):
            acc = acc + w[j] * full[W + i - j]
        out[i] = acc
    return out


def modal_iir(g: np.ndarray, s_prev: np.ndarray, lam, beta, c):
    """Diagonal modal IIR scan keeping every per-position state.

    g [P][d]; s_prev [d][N] is the committed state s_{-1}.  For each position i:
    s_i = lam * s_{i-1} + beta * g_i (broadcast over the N poles), and the
    readout y_i = sum_n c * s_i.  Returns (s [P][d][N], y [P][d]).  The states
    s_0..s_gamma are kept so that slicing can select s_k (EvSpark digest,
    Figure 1(d): "retain IIR state s3").
    """
    gg = as_f64(g)
    lam, beta, c = as_f64(lam), as_f64(beta), as_f64(c)
    s = as_f64(s_prev).copy()
    P, d = gg.shape
    S = np.zeros((P,) + s.shape)
    Y = np.zeros((P, d))
    for i in range(P):
        s = lam * s + beta * gg[i][:, None]
        S[i] = s
        Y[i] = (c * s).sum(axis=1)
    return S, Y


def block_attention(q, k_blk, v_blk, k_blocks, v_blocks) -> np.ndarray:
    """Causal block attention of P block queries over the committed KV prefix.

    q, k_blk, v_blk: [P][H][Dh] block rows; k_blocks / v_blocks: committed rows
    as a list of [H][n][Dh] arrays.  Query i attends to all committed keys and
    to block keys 0..i (itself included); scores are scaled by 1/sqrt(Dh); the
    softmax is the explicit full matrix over those keys.  Returns o [P][H][Dh].
    """
    qq = as_f64(q)
    kb = as_f64(k_blk)
    vb = as_f64(v_blk)
    P, H, Dh = qq.shape
    o = np.zeros((P, H, Dh))
    scale = 1.0 / math.sqrt(Dh)
    for h in range(H):
        keys = np.concatenate([as_f64(b[h]) for b in k_blocks] + [kb[:, h, :]], axis=0)
        vals = np.concatenate([as_f64(b[h]) for b in v_blocks] + [vb[:, h, :]], axis=0)
        L = keys.shape[0] - P
        scores = (keys @ qq[:, h, :].T) * scale          # [L+P][P]
        for i in range(P):                                # block key j is visible to query i iff j <= i
            scores[L + i + 1:, i] = -np.inf
        m = scores.max(axis=0)
        w = np.exp(scores - m[None, :])
        w = w / w.sum(axis=0)[None, :]
        o[:, h, :] = w.T @ vals
    return o


def verify_block(layer: Layer, st: SeqState, x, q, k, v):
    """One initial-state block forward over the anchor and gamma drafts.

    The EvSpark digest (Interpretation) verifies a whole block in a single
    forward from the committed state, without mutating it; the block's
    intermediate values are what slicing later selects from.

    x [P][d], q/k/v [P][H][Dh].  Returns dict f [P][d] (outer-FIR inputs),
    s [P][d][N] (IIR states), y [P][d], o [P][H][Dh].
    """
    f = depthwise_fir(x, st.short_win, layer.w_short)
    g = depthwise_fir(f, st.outer_win, layer.w_outer)
    s, y = modal_iir(g, st.iir, layer.lam, layer.beta, layer.c)
    o = block_attention(q, k, v, st.k_blocks, st.v_blocks)
    return {"f": f, "s": s, "y": y, "o": o}
