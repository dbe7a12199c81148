"""Oracle: the drafter trunk and its serial Markov-biased sampling (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The EvSpark digest (Figure 1(b); Interpretation) describes the drafter: a
projected window of up to W = 64 target states forms the K/V prefix of each
of two causal attention layers of width d = 1024; anchor and mask
embeddings give all draft logits in one trunk pass; input and output
embeddings are tied; a previous-token full-matrix Markov bias then supports
serial sampling; a confidence head does not control decoding (left out).
The pages print no equations; the plain reading used here:

* hw = window (target states, [W][d_t]) @ W_proj, rounded to bf16;
* block rows: the anchor's embedding row, then gamma - 1 copies of the mask
  embedding (one row per draft: row i gives the logits of draft t_{i+1});
* each trunk layer (pre-norm residual): a = RMSNorm(h); (q, k, v) = a W_qkv
  for the block rows and (k, v) = RMSNorm(hw) W_qkv for the window rows;
  causal block attention with the window as committed prefix; h <- h + o W_o;
  then h <- h + SiLU(RMSNorm(h) W_up) W_down;
* logits z = RMSNorm(h) E^T (fp32, E the tied embedding);
* serial sampling: prev = anchor; draft m uses the fp32 logits
  z[m-1] + B[prev] (B the Markov bias, [V][V]); its token is the inverse-CDF
  draw of softmax(logits / T) with the uniform u_m, under the acceptance
  rule's conventions; those biased logits are the distribution the draft was
  sampled from (the q that acceptance needs);
* bf16 rounding points as on the device: a, q/k/v, o, the MLP activation,
  every new h, hw and the final RMSNorm output.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from .acceptance import _inverse_cdf, _softmax
from .layer import as_f64, block_attention
from .linear import linear, rmsnorm
from .model import bf16_round


@dataclass
class TrunkLayer:
    g1: np.ndarray          # [d]
    w_qkv: np.ndarray       # [d][3d]
    w_o: np.ndarray         # [d][d]
    g2: np.ndarray          # [d]
    w_up: np.ndarray        # [d][F]
    w_down: np.ndarray      # [F][d]


@dataclass
class Drafter:
    w_proj: np.ndarray      # [d_t][d]
    emb: np.ndarray         # [V][d] tied input / output embedding
    mask: np.ndarray        # [d]
    markov: np.ndarray      # [V][V] fp32: B[prev][next]
    layers: List[TrunkLayer]
    g_f: np.ndarray         # [d]
    heads: int
    eps: float


def _silu(x):
    return x / (1.0 + np.exp(-x))


def draft_logits(dr: Drafter, window, anchor: int, gamma: int, rounding: bool = True) -> np.ndarray:
    """Trunk pass for one sequence: z [gamma][V] (row i: logits of draft t_{i+1}, before the bias)."""
    rnd = bf16_round if rounding else as_f64
    d = dr.emb.shape[1]
    H = dr.heads
    Dh = d // H
    hw = rnd(linear(window, dr.w_proj))
    h = np.concatenate([as_f64(dr.emb[anchor])[None, :], np.repeat(as_f64(dr.mask)[None, :], gamma - 1, axis=0)])
    for L in dr.layers:
        a = rnd(rmsnorm(h, L.g1, dr.eps))
        aw = rnd(rmsnorm(hw, L.g1, dr.eps))
        qkv = rnd(linear(a, L.w_qkv))
        kvw = rnd(linear(aw, L.w_qkv))
        P, W = h.shape[0], hw.shape[0]
        q = qkv[:, :d].reshape(P, H, Dh)
        k = qkv[:, d:2 * d].reshape(P, H, Dh)
        v = qkv[:, 2 * d:].reshape(P, H, Dh)
        kw = kvw[:, d:2 * d].reshape(W, H, Dh).transpose(1, 0, 2)
        vw = kvw[:, 2 * d:].reshape(W, H, Dh).transpose(1, 0, 2)
        o = rnd(block_attention(q, k, v, [kw], [vw]).reshape(P, d))
        h = rnd(linear(o, L.w_o, h))
        m = rnd(_silu(linear(rnd(rmsnorm(h, L.g2, dr.eps)), L.w_up)))
        h = rnd(linear(m, L.w_down, h))
    hf = rnd(rmsnorm(h, dr.g_f, dr.eps))
    return linear(hf, as_f64(dr.emb).T)


def draft_sample(z, markov, anchor: int, u, temperature: float = 1.0):
    """Serial sampling with the previous-token bias: (drafts [gamma], biased logits [gamma][V] fp32, margins)."""
    zz = np.asarray(z, np.float32)
    B = np.asarray(markov, np.float32)
    gamma, V = zz.shape
    drafts = np.zeros(gamma, np.int32)
    out = np.zeros((gamma, V), np.float32)
    margins = np.zeros(gamma)
    prev = int(anchor)
    for m in range(gamma):
        logit = zz[m] + B[prev]                      # fp32 addition
        out[m] = logit
        t, margins[m] = _inverse_cdf(_softmax(logit, temperature), float(u[m]))
        drafts[m] = t
        prev = t
    return drafts, out, margins
