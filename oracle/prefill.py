"""Oracle: prefill of a prompt into the committed state (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The step before the verify hot path: a prompt of T positions is run through
the conv/recurrent path and its K/V rows are appended, leaving the committed
state the first verify starts from.  By the block-forward contract (EvSpark
digest, Interpretation: one initial-state block forward plus slicing equals
sequential decoding) this is a block forward over all T positions followed by
a slice at T-1, restricted to the state: the FIR windows, the IIR state and
the KV prefix.  The prompt's attention outputs are not part of the state and
are not computed here.

``depthwise_fir_long`` is the same causal convolution as ``depthwise_fir``
written with ``numpy.convolve`` (a library convolution primitive) so that
long prompts finish in seconds; both are pinned against each other.
"""
from __future__ import annotations

import numpy as np

from .layer import Layer, SeqState, as_f64, depthwise_fir


def depthwise_fir_long(block, window, taps) -> np.ndarray:
    """out_i[ch] = sum_{j<T} taps[j][ch] * in[i-j][ch] over [window ; block], via numpy.convolve."""
    blk = as_f64(block)
    win = as_f64(window)
    w = as_f64(taps)
    P, d = blk.shape
    W = win.shape[0]
    full = np.concatenate([win, blk], axis=0)
    out = np.empty((P, d))
    for ch in range(d):
        out[:, ch] = np.convolve(full[:, ch], w[:, ch])[W:W + P]
    return out


def iir_scan(g, s_prev, lam, beta, c):
    """s_i = lam * s_{i-1} + beta * g_i, y_i = sum_n c * s_i; returns (s_last, y) without keeping every s_i."""
    gg = as_f64(g)
    lam, beta, c = as_f64(lam), as_f64(beta), as_f64(c)
    s = as_f64(s_prev).copy()
    y = np.zeros(gg.shape)
    for i in range(gg.shape[0]):
        s = lam * s + beta * gg[i][:, None]
        y[i] = (c * s).sum(axis=1)
    return s, y


def _last_rows(window, rows):
    W = window.shape[0]
    if W == 0:
        return np.zeros((0,) + window.shape[1:])
    both = np.concatenate([as_f64(window), as_f64(rows)], axis=0)
    return both[both.shape[0] - W:]


def prefill_state(layer: Layer, st: SeqState, x, k_rows, v_rows, long: bool = False):
    """Committed state after the T prompt positions x [T][d], k/v [T][H][Dh]; also y [T][d].

    Returns (new SeqState, y).  ``long`` selects the numpy.convolve FIR.
    """
    fir = depthwise_fir_long if long else depthwise_fir
    f = fir(x, st.short_win, layer.w_short)
    g = fir(f, st.outer_win, layer.w_outer)
    s_last, y = iir_scan(g, st.iir, layer.lam, layer.beta, layer.c)
    kb = np.ascontiguousarray(np.asarray(k_rows).transpose(1, 0, 2))
    vb = np.ascontiguousarray(np.asarray(v_rows).transpose(1, 0, 2))
    new = SeqState(short_win=_last_rows(st.short_win, x), outer_win=_last_rows(st.outer_win, f), iir=s_last,
                   k_blocks=list(st.k_blocks) + [kb], v_blocks=list(st.v_blocks) + [vb])
    return new, y
