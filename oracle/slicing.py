"""Oracle: state slicing to the accepted index, and the sequential reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

EvSpark digest, Figure 1(d): after k drafts are accepted the state returns to
block index k -- the readable KV prefix grows by the k+1 consumed positions,
the FIR windows keep the last inputs up to position k, and the IIR state
becomes s_k.  Nothing is recomputed (no replay).  The sequential reference
(one position per forward) is the replay that slicing replaces
(Interpretation: a second target forward).
"""
from __future__ import annotations

import numpy as np

from .layer import Layer, SeqState, as_f64, verify_block


def _last_rows(window: np.ndarray, new_rows: np.ndarray) -> np.ndarray:
    W = window.shape[0]
    if W == 0:
        return window.copy()
    both = np.concatenate([as_f64(window), as_f64(new_rows)], axis=0)
    return both[both.shape[0] - W:]


def slice_state(st: SeqState, x, fwd, k_blk, v_blk, k: int) -> SeqState:
    """Commit block positions 0..k of a verified block into a new state.

    x [P][d] block inputs; fwd is ``verify_block``'s result (f, s);
    k_blk / v_blk [P][H][Dh].  Returns the new SeqState:
      short window <- last Ts-1 rows of [window ; x_0..x_k]
      outer window <- last To-1 rows of [window ; f_0..f_k]   (outer-FIR inputs u)
      IIR state    <- s_k
      KV prefix    <- prefix followed by block rows 0..k
    """
    kb = np.ascontiguousarray(np.asarray(k_blk)[: k + 1].transpose(1, 0, 2))   # [H][k+1][Dh]
    vb = np.ascontiguousarray(np.asarray(v_blk)[: k + 1].transpose(1, 0, 2))
    return SeqState(
        short_win=_last_rows(st.short_win, np.asarray(x)[: k + 1]),
        outer_win=_last_rows(st.outer_win, fwd["f"][: k + 1]),
        iir=np.array(fwd["s"][k], dtype=np.float64),
        k_blocks=list(st.k_blocks) + [kb],
        v_blocks=list(st.v_blocks) + [vb],
    )


def sequential_steps(layer: Layer, st: SeqState, x, q, k, v, count: int):
    """``count`` single-position forwards, each committed before the next.

    Each step is a block forward with gamma = 0 followed by a slice at 0.
    Returns (state, outputs) with outputs stacked like a block forward's.
    """
    outs = {"f": [], "s": [], "y": [], "o": []}
    cur = st
    for i in range(count):
        fwd = verify_block(layer, cur, x[i:i + 1], q[i:i + 1], k[i:i + 1], v[i:i + 1])
        for key in outs:
            outs[key].append(fwd[key][0])
        cur = slice_state(cur, x[i:i + 1], fwd, k[i:i + 1], v[i:i + 1], 0)
    return cur, {key: np.stack(val) for key, val in outs.items()}
