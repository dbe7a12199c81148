"""Oracle: a stack of full hybrid layers verified as one block, sliced, and stepped (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The target of the pages is a StripedHyena2 model (EvSpark digest, Synopsis and
Figure 1(a): Evo2, a hybrid convolutional-recurrent-attention model) whose
inference state falls into three classes -- FIR windows, modal IIR states
and KV caches (Interpretation; Figure 1(d)).  The pages print no layer
equations; the plainest reading of a striped Hyena / attention stack is used:

* the residual stream x [P][d] enters every layer; a = RMSNorm(x) (gain g);
  the mixer output goes through an output projection and is added to x;
* Hyena mixer: z = a W_in, split into three streams (z_q, z_k, z_v) of d
  channels; a short depthwise FIR of Ts taps runs on all 3d channels (its
  window holds the last Ts-1 rows of z); u = zk_hat * zv_hat; the long
  operator h = op(u) is either an explicit FIR of Tl taps (kind "fir": the
  short-explicit and medium-regularised layers; its window holds the last
  Tl-1 rows of u -- the "outer-FIR inputs" of Figure 1(d)) or a diagonal
  modal IIR (kind "iir": the long-implicit layers, s_i = lam s_{i-1} + beta
  u_i, h_i = sum_n c s_i, every s_i kept); y = zq_hat * h;
* attention mixer: (q, k, v) = a W_qkv, heads of Dh, causal block attention
  over the committed KV prefix; y = o;
* rounding points (``rounding=True``, as the device path stores them): a,
  y, the new x, and the attention layer's q/k/v are rounded to bf16 (round
  to nearest even); z, the FIR outputs, u, h and s are not rounded;
* feature buffer (the drafter's window of target states, Figure 1(b)(d)):
  the residual stream after layer ``feature_layer`` for the last W
  committed positions, sliced with the rest of the state.

Every step is one of the pinned single-layer pieces (depthwise FIR, modal
IIR, block attention, linear, rmsnorm) or an elementwise product.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

from .layer import as_f64, block_attention, depthwise_fir, modal_iir
from .linear import linear, rmsnorm


def bf16_round(a) -> np.ndarray:
    """Round each value to the nearest bf16 (8 significant bits), ties to even."""
    a = as_f64(a)
    m, e = np.frexp(a)                     # a = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)   # numpy rounds halves to even


@dataclass
class Mixer:
    kind: str                              # "fir" | "iir" | "attn"
    g: np.ndarray                          # [d] RMSNorm gain
    w_in: np.ndarray                       # [d][3d]
    w_out: np.ndarray                      # [d][d]
    w_short: np.ndarray = None             # [Ts][3d]  (Hyena)
    w_long: np.ndarray = None              # [Tl][d]   (fir)
    lam: np.ndarray = None                 # [d][N]    (iir)
    beta: np.ndarray = None
    c: np.ndarray = None


@dataclass
class Model:
    mixers: List[Mixer]
    d: int
    heads: int
    head_dim: int
    eps: float
    feature_layer: int
    feature_window: int


@dataclass
class LayerState:
    short_win: np.ndarray = None           # [Ts-1][3d]
    long_win: np.ndarray = None            # [Tl-1][d]
    iir: np.ndarray = None                 # [d][N]
    k_blocks: list = field(default_factory=list)   # attention: committed rows, [H][n][Dh] arrays
    v_blocks: list = field(default_factory=list)


@dataclass
class ModelState:
    layers: List[LayerState]
    feature: np.ndarray                    # [W][d]


def _rnd(a, rounding):
    return bf16_round(a) if rounding else as_f64(a)


def model_verify_block(model: Model, st: ModelState, x, rounding: bool = True) -> Dict:
    """One block forward over P rows from the committed state (nothing is modified).

    Returns {"x": [L+1][P][d] residual streams (x[0] = input), "layers": per layer
    the tensors slicing needs ("z" [3][P][d]; "u" [P][d] or "s" [P][d][N];
    attention: "k", "v" [P][H][Dh]) and, for Hyena layers, the short-FIR
    outputs "zh" [3][P][d]}.
    """
    d, H, Dh = model.d, model.heads, model.head_dim
    xs = [as_f64(x)]
    kept = []
    for mx, ls in zip(model.mixers, st.layers):
        xl = xs[-1]
        a = _rnd(rmsnorm(xl, mx.g, model.eps), rounding)
        z = linear(a, mx.w_in)                                   # [P][3d]
        P = z.shape[0]
        if mx.kind == "attn":
            z = _rnd(z, rounding)
            q = z[:, :d].reshape(P, H, Dh)
            k = z[:, d:2 * d].reshape(P, H, Dh)
            v = z[:, 2 * d:].reshape(P, H, Dh)
            y = block_attention(q, k, v, ls.k_blocks, ls.v_blocks).reshape(P, d)
            rec = {"z": np.stack([z[:, :d], z[:, d:2 * d], z[:, 2 * d:]]), "k": k, "v": v}
        else:
            zh = depthwise_fir(z, ls.short_win, mx.w_short)           # featurizer on all 3d channels
            zq, zk, zv = zh[:, :d], zh[:, d:2 * d], zh[:, 2 * d:]
            u = zk * zv
            if mx.kind == "fir":
                h = depthwise_fir(u, ls.long_win, mx.w_long)
                rec = {"u": u}
            else:
                S, h = modal_iir(u, ls.iir, mx.lam, mx.beta, mx.c)
                rec = {"s": S}
            y = zq * h
            rec["z"] = np.stack([z[:, :d], z[:, d:2 * d], z[:, 2 * d:]])
            rec["zh"] = np.stack([zq, zk, zv])
        y = _rnd(y, rounding)
        xs.append(_rnd(linear(y, mx.w_out, xl), rounding))
        kept.append(rec)
    return {"x": np.stack(xs), "layers": kept}


def _last_rows(window, rows):
    W = window.shape[0]
    both = np.concatenate([as_f64(window), as_f64(rows)], axis=0)
    return both[both.shape[0] - W:]


def model_slice_state(model: Model, st: ModelState, fwd: Dict, k: int) -> ModelState:
    """State after accepting block rows 0..k (EvSpark digest, Figure 1(d), per layer)."""
    new_layers = []
    for mx, ls, rec in zip(model.mixers, st.layers, fwd["layers"]):
        if mx.kind == "attn":
            kb = np.ascontiguousarray(as_f64(rec["k"][: k + 1]).transpose(1, 0, 2))
            vb = np.ascontiguousarray(as_f64(rec["v"][: k + 1]).transpose(1, 0, 2))
            new_layers.append(LayerState(k_blocks=list(ls.k_blocks) + [kb], v_blocks=list(ls.v_blocks) + [vb]))
            continue
        z = rec["z"][:, : k + 1]                                  # [3][k+1][d]
        zrows = np.concatenate([z[0], z[1], z[2]], axis=1)        # [k+1][3d], the in-projection rows
        nl = LayerState(short_win=_last_rows(ls.short_win, zrows))
        if mx.kind == "fir":
            nl.long_win = _last_rows(ls.long_win, rec["u"][: k + 1])
        else:
            nl.iir = as_f64(rec["s"][k]).copy()
        new_layers.append(nl)
    feat_rows = fwd["x"][model.feature_layer + 1][: k + 1]
    return ModelState(layers=new_layers, feature=_last_rows(st.feature, feat_rows))


def model_sequential_steps(model: Model, st: ModelState, x, count: int, rounding: bool = True):
    """count single-position steps (a one-row block forward, then a slice at 0): the replay path."""
    outs = []
    cur = st
    for i in range(count):
        fwd = model_verify_block(model, cur, as_f64(x)[i: i + 1], rounding)
        outs.append(fwd["x"][-1][0])
        cur = model_slice_state(model, cur, fwd, 0)
    return cur, np.stack(outs)
