"""Seeded synthetic inputs for the hybrid conv/IIR/attention verify path.

This module only draws random numbers and arranges them into arrays.  It
holds none of the method's arithmetic (no FIR, no IIR step, no softmax, no
attention, no acceptance rule), so that the fp64 oracle and the HIP path can
both be fed from it without sharing any computation.

Workloads follow the five operating points of the EvSpark digest (Synopsis
and Perspective: 7B-scale layers, 51k-262k context, batching, multiple
candidates, sustained generation) as fixed synthetic shapes:

* ``tiny``  fp32 layer: d=64, 3/7 FIR taps, 16 poles, 1 head x 64, L=256, gamma=6
* ``mid8k``  d=4096, bf16, 3/128 taps, 16 poles, 32 heads x 128, L=8192, gamma=12, sampling
* ``long262k``  the mid8k layer at L=262144, gamma=12 (``long262k``) or gamma=6 (``long262k_g6``), greedy
* ``multi4x4``  4 sequences x 4 candidates, ragged L in {16384, 32768, 51200, 65536}
* ``wide131k``  d=8192, 64 heads x 128, L=131072, gamma=12, 256 sustained rounds

Distributions (variance readings): FIR taps N(0, 1/taps); poles U(0.5, 0.99);
input and readout gains N(0, 1/16); activations and KV N(0, 1); logits N(0, 2).
bf16 values are produced by round-to-nearest-even from fp32 and are handed to
both sides as raw 16-bit patterns (``numpy.uint16``).

Random streams are independent torch CPU generators keyed by
``(config id, stream id, round)``; the large KV prefixes can instead be drawn
on a GPU with torch's device generator (``kv_prefix(..., device="cuda")``),
the host side then receives a copy of the very same bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

# fixed stream ids (part of every seed)
_S_WSHORT, _S_WOUTER, _S_LAMBDA, _S_BETA, _S_C = 1, 2, 3, 4, 5
_S_EX, _S_EQ, _S_EK, _S_EV = 10, 11, 12, 13
_S_SWIN, _S_OWIN, _S_IIR = 20, 21, 22
_S_KPRE, _S_VPRE = 30, 31
_S_TOK, _S_ZT, _S_ZD, _S_GUMBEL, _S_U, _S_GEOM = 40, 41, 42, 43, 44, 45
_S_NEEDLE = 50
_S_PROMPT = 60
_S_DENSE = 70


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    d: int
    taps_short: int
    taps_outer: int
    poles: int
    heads: int
    head_dim: int
    kv_lens: tuple          # committed prefix length per sequence
    gamma: int
    nc: int = 1             # candidate blocks per sequence
    vocab: int = 512
    act: str = BF16
    mode: str = "sample"    # "greedy" or "sample"
    temperature: float = 1.0
    rounds: int = 1

    @property
    def nb(self) -> int:
        return len(self.kv_lens)

    @property
    def P(self) -> int:
        return self.gamma + 1

    @property
    def max_kv_len(self) -> int:
        return max(self.kv_lens)

    def kv_cap(self, extra_rounds: Optional[int] = None) -> int:
        r = self.rounds if extra_rounds is None else extra_rounds
        need = self.max_kv_len + (r + 1) * self.P
        return (need + 31) // 32 * 32


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, d=64, taps_short=3, taps_outer=7, poles=16, heads=1, head_dim=64,
                 kv_lens=(256,), gamma=6, act=F32, mode="sample"),
    "mid8k": Config("mid8k", 2, d=4096, taps_short=3, taps_outer=128, poles=16, heads=32, head_dim=128,
                 kv_lens=(8192,), gamma=12, act=BF16, mode="sample"),
    "long262k": Config("long262k", 3, d=4096, taps_short=3, taps_outer=128, poles=16, heads=32, head_dim=128,
                 kv_lens=(262144,), gamma=12, act=BF16, mode="greedy"),
    "long262k_g6": Config("long262k_g6", 6, d=4096, taps_short=3, taps_outer=128, poles=16, heads=32, head_dim=128,
                   kv_lens=(262144,), gamma=6, act=BF16, mode="greedy"),
    "multi4x4": Config("multi4x4", 4, d=4096, taps_short=3, taps_outer=128, poles=16, heads=32, head_dim=128,
                 kv_lens=(16384, 32768, 51200, 65536), gamma=12, nc=4, act=BF16, mode="sample"),
    "wide131k": Config("wide131k", 5, d=8192, taps_short=3, taps_outer=128, poles=16, heads=64, head_dim=128,
                 kv_lens=(131072,), gamma=12, act=BF16, mode="greedy", rounds=256),
}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity variants)."""
    return dataclasses.replace(cfg, **kw)


# ---------------------------------------------------------------- generators

def _gen(cfg: Config, stream: int, rnd: int = 0, seed: int = 0) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(((seed * 1000 + cfg.cfg_id) * 100 + stream) * 100003 + rnd)
    return g


def bf16_bits(a: torch.Tensor) -> np.ndarray:
    """fp32 tensor -> bf16 bit patterns (round to nearest even) as uint16."""
    return a.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _act(cfg: Config, t: torch.Tensor) -> np.ndarray:
    t = t.to(torch.float32)
    return bf16_bits(t) if cfg.act == BF16 else t.numpy().astype(np.float32)


def _normal(cfg, stream, shape, std=1.0, rnd=0, seed=0) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(cfg, stream, rnd, seed), dtype=torch.float32) * std


# ---------------------------------------------------------------- layer

def make_layer(cfg: Config, seed: int = 0) -> Dict[str, np.ndarray]:
    d, N = cfg.d, cfg.poles
    lam = torch.rand((d, N), generator=_gen(cfg, _S_LAMBDA, 0, seed), dtype=torch.float64)
    lam = (0.5 + 0.49 * lam).to(torch.float32)
    return {
        "w_short": _normal(cfg, _S_WSHORT, (cfg.taps_short, d), 1.0 / math.sqrt(cfg.taps_short), seed=seed).numpy(),
        "w_outer": _normal(cfg, _S_WOUTER, (cfg.taps_outer, d), 1.0 / math.sqrt(cfg.taps_outer), seed=seed).numpy(),
        "lam": lam.numpy(),
        "beta": _normal(cfg, _S_BETA, (d, N), 0.25, seed=seed).numpy(),
        "c": _normal(cfg, _S_C, (d, N), 0.25, seed=seed).numpy(),
    }


def make_tables(cfg: Config, seed: int = 0) -> Dict[str, np.ndarray]:
    """Token-keyed input tables: block inputs are rows of these tables."""
    V, d, H, Dh = cfg.vocab, cfg.d, cfg.heads, cfg.head_dim
    return {
        "E_x": _act(cfg, _normal(cfg, _S_EX, (V, d), seed=seed)),
        "E_q": _act(cfg, _normal(cfg, _S_EQ, (V, H, Dh), seed=seed)),
        "E_k": _act(cfg, _normal(cfg, _S_EK, (V, H, Dh), seed=seed)),
        "E_v": _act(cfg, _normal(cfg, _S_EV, (V, H, Dh), seed=seed)),
    }


def make_state_small(cfg: Config, seed: int = 0) -> Dict[str, np.ndarray]:
    """Committed FIR windows and IIR state (the KV prefix is drawn separately)."""
    nb, d, N = cfg.nb, cfg.d, cfg.poles
    return {
        "short_win": _act(cfg, _normal(cfg, _S_SWIN, (nb, cfg.taps_short - 1, d), seed=seed)),
        "outer_win": _normal(cfg, _S_OWIN, (nb, cfg.taps_outer - 1, d), seed=seed).numpy(),
        "iir": _normal(cfg, _S_IIR, (nb, d, N), 0.5, seed=seed).numpy(),
    }


def kv_prefix(cfg: Config, b: int, which: str, seed: int = 0, device: str = "cpu",
              length: Optional[int] = None) -> torch.Tensor:
    """Committed KV prefix of sequence ``b``: [H][L][Dh] ~ N(0,1) in act dtype.

    Returns a torch tensor (bf16 or fp32) on ``device``.  On a GPU the values
    come from torch's device generator; on the CPU from torch's CPU generator.
    """
    L = cfg.kv_lens[b] if length is None else length
    stream = _S_KPRE if which == "k" else _S_VPRE
    s = ((seed * 1000 + cfg.cfg_id) * 100 + stream) * 100003 + 7 * b + 1
    g = torch.Generator(device=device)
    g.manual_seed(s)
    out_dtype = torch.bfloat16 if cfg.act == BF16 else torch.float32
    out = torch.empty((cfg.heads, L, cfg.head_dim), dtype=out_dtype, device=device)
    for h in range(cfg.heads):  # one head at a time bounds the fp32 temporary
        out[h] = torch.randn((L, cfg.head_dim), generator=g, device=device, dtype=torch.float32).to(out_dtype)
    return out


def prompt(cfg: Config, T: int, seed: int = 0, device: str = "cpu"):
    """A prompt of T positions for every sequence: x [nb][T][d], k, v [nb][T][H][Dh] ~ N(0, 1), act dtype.

    Drawn with torch's generator on ``device`` (the host receives copies of the same bits).
    """
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000 + cfg.cfg_id) * 100 + _S_PROMPT) * 100003 + T)
    out_dtype = torch.bfloat16 if cfg.act == BF16 else torch.float32
    shapes = {"x": (cfg.nb, T, cfg.d), "k": (cfg.nb, T, cfg.heads, cfg.head_dim), "v": (cfg.nb, T, cfg.heads, cfg.head_dim)}
    out = {}
    for name, shape in shapes.items():
        t = torch.empty(shape, dtype=out_dtype, device=device)
        for b in range(cfg.nb):
            t[b] = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32).to(out_dtype)
        out[name] = t
    return out


def dense(shape, std: float, tag: int, seed: int = 0, device: str = "cpu") -> torch.Tensor:
    """A seeded N(0, std^2) bf16 tensor (weights, activations of the dense projections)."""
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000 + tag) * 100 + _S_DENSE) * 100003 + int(np.prod(shape)) % 100003)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def needle_positions(cfg: Config, b: int, count: int = 4, seed: int = 0) -> np.ndarray:
    """Prefix rows where a key is replaced by a scaled copy of a block query."""
    L = cfg.kv_lens[b]
    g = _gen(cfg, _S_NEEDLE, b, seed)
    return torch.randint(0, max(L, 1), (count,), generator=g).numpy()


# ---------------------------------------------------------------- tokens, logits, uniforms

def gather_block(cfg: Config, tables: Dict[str, np.ndarray], tokens: np.ndarray) -> Dict[str, np.ndarray]:
    """Block inputs from token ids ``tokens`` [nb][nc][P]: x, q, k, v rows of the tables."""
    return {
        "x": tables["E_x"][tokens],   # [nb][nc][P][d]
        "q": tables["E_q"][tokens],   # [nb][nc][P][H][Dh]
        "k": tables["E_k"][tokens],
        "v": tables["E_v"][tokens],
    }


def anchors(cfg: Config, rnd: int = 0, seed: int = 0) -> np.ndarray:
    return torch.randint(0, cfg.vocab, (cfg.nb,), generator=_gen(cfg, _S_TOK, rnd, seed)).numpy().astype(np.int32)


def logits(cfg: Config, stream: str, rows: int, rnd: int = 0, seed: int = 0) -> np.ndarray:
    """[nb][nc][rows][V] fp32 logits ~ N(0, 2)."""
    sid = _S_ZT if stream == "target" else _S_ZD
    return _normal(cfg, sid, (cfg.nb, cfg.nc, rows, cfg.vocab), math.sqrt(2.0), rnd, seed).numpy()


def uniforms(cfg: Config, rnd: int = 0, seed: int = 0) -> np.ndarray:
    """[nb][nc][P] fp64 uniforms in [0, 1): r_1..r_gamma then r*."""
    g = _gen(cfg, _S_U, rnd, seed)
    return torch.rand((cfg.nb, cfg.nc, cfg.P), generator=g, dtype=torch.float64).numpy()


def gumbel_drafts(cfg: Config, draft_logits: np.ndarray, rnd: int = 0, seed: int = 0) -> np.ndarray:
    """Draft tokens sampled from softmax(draft_logits / T) by the Gumbel-max trick.

    ``argmax(z / T + G)`` with G i.i.d. standard Gumbel is an exact sample of the
    categorical distribution softmax(z / T); no probabilities are formed here.
    """
    g = _gen(cfg, _S_GUMBEL, rnd, seed)
    u = torch.rand(draft_logits.shape, generator=g, dtype=torch.float64).numpy()
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    gum = -np.log(-np.log(u))
    return np.argmax(draft_logits.astype(np.float64) / cfg.temperature + gum, axis=-1).astype(np.int32)


def prefix_row(cfg: Config, rnd: int, seed: int, kind: int, b: int, prefix, scale: float = math.sqrt(2.0)):
    """A seeded N(0, scale^2) logit row keyed by (kind, sequence, drafted prefix): kind 0 = the target's
    row after the prefix, kind 1 = the drafter's."""
    g = np.random.default_rng([cfg.cfg_id, seed, rnd, kind, b, len(prefix)] + [int(t) for t in prefix])
    return (g.standard_normal(cfg.vocab) * scale).astype(np.float32)


def prefix_keyed_round(cfg: Config, rnd: int = 0, seed: int = 0, scale: float = math.sqrt(2.0)):
    """Sampling inputs whose logit rows are a seeded function of (sequence, prefix).

    Candidates of a sequence that share a draft prefix get the same target and
    draft rows at the next position, and each candidate's drafts are
    independent Gumbel-max draws from its draft rows -- what several
    candidate blocks drafted from one anchor look like.  Returns
    (target_logits [nb][nc][P][V], draft_logits [nb][nc][gamma][V],
    drafts [nb][nc][gamma], uniforms [nb][nc][P]).
    """
    nb, nc, gam, V = cfg.nb, cfg.nc, cfg.gamma, cfg.vocab

    def row(kind, b, prefix):
        return prefix_row(cfg, rnd, seed, kind, b, prefix, scale)

    noise = np.random.default_rng([cfg.cfg_id, seed, rnd, 7]).random((nb, nc, max(gam, 1), V))
    noise = np.clip(noise, 1e-300, 1.0 - 1e-16)
    zt = np.empty((nb, nc, gam + 1, V), np.float32)
    zd = np.empty((nb, nc, gam, V), np.float32)
    drafts = np.empty((nb, nc, gam), np.int32)
    for b in range(nb):
        for c in range(nc):
            pre = []
            for i in range(gam):
                zt[b, c, i] = row(0, b, pre)
                zd[b, c, i] = row(1, b, pre)
                gum = -np.log(-np.log(noise[b, c, i]))
                drafts[b, c, i] = int(np.argmax(zd[b, c, i].astype(np.float64) / cfg.temperature + gum))
                pre.append(int(drafts[b, c, i]))
            zt[b, c, gam] = row(0, b, pre)
    return zt, zd, drafts, uniforms(cfg, rnd, seed)


def geometric_agreement(cfg: Config, rnd: int = 0, seed: int = 0, p_continue: float = 0.7,
                        forced_len: Optional[Sequence[int]] = None):
    """Greedy workload: drafts agree with the target argmax for a Geometric(0.7) prefix.

    Returns (drafts [nb][nc][gamma] int32, target_logits [nb][nc][P][V] fp32, lengths).
    Agreement is planted, not measured: row m-1 of the target logits gets a
    logit of +100 at draft t_m for m <= Lg (N(0,2) logits never come near it),
    and row Lg gets -100 at draft t_{Lg+1}, so that draft cannot be the argmax.
    """
    nb, nc, gam, V = cfg.nb, cfg.nc, cfg.gamma, cfg.vocab
    g = _gen(cfg, _S_GEOM, rnd, seed)
    drafts = torch.randint(0, V, (nb, nc, gam), generator=g).numpy().astype(np.int32)
    zt = logits(cfg, "target", cfg.P, rnd, seed)
    lens = np.zeros((nb, nc), dtype=np.int32)
    u = torch.rand((nb, nc, gam), generator=g, dtype=torch.float64).numpy()
    for b in range(nb):
        for c in range(nc):
            if forced_len is not None:
                n = int(forced_len[b * nc + c])
            else:
                n = 0
                while n < gam and u[b, c, n] < p_continue:
                    n += 1
            lens[b, c] = n
            for m in range(1, n + 1):
                zt[b, c, m - 1, drafts[b, c, m - 1]] = 100.0
            if n < gam:
                zt[b, c, n, drafts[b, c, n]] = -100.0
    return drafts, zt, lens


def block_tokens(anchor: np.ndarray, drafts: np.ndarray) -> np.ndarray:
    """[nb] anchors and [nb][nc][gamma] drafts -> [nb][nc][P] block tokens."""
    nb, nc, gam = drafts.shape
    t = np.empty((nb, nc, gam + 1), dtype=np.int32)
    t[:, :, 0] = anchor[:, None]
    t[:, :, 1:] = drafts
    return t


def round_inputs(cfg: Config, anchor: np.ndarray, rnd: int = 0, seed: int = 0,
                 forced_len: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Everything one verify/accept round needs besides layer, state and tables."""
    if cfg.mode == "greedy":
        drafts, zt, lens = geometric_agreement(cfg, rnd, seed, forced_len=forced_len)
        zd = None
        u = None
    elif cfg.mode == "recursive":
        zt, zd, drafts, u = prefix_keyed_round(cfg, rnd, seed)
        lens = None
    else:
        zt = logits(cfg, "target", cfg.P, rnd, seed)
        zd = logits(cfg, "draft", cfg.gamma, rnd, seed)
        drafts = gumbel_drafts(cfg, zd, rnd, seed)
        u = uniforms(cfg, rnd, seed)
        lens = None
    return {"drafts": drafts, "target_logits": zt, "draft_logits": zd, "uniforms": u,
            "tokens": block_tokens(anchor, drafts), "planted_len": lens}


# ---------------------------------------------------------------- token trees

def trie_of(tokens: np.ndarray):
    """The token tree of several candidate blocks that share the anchor: one node per distinct
    prefix.  tokens [nc][P] (position 0 = the anchor).  Nodes are numbered in order of first
    appearance (candidate-major, position-minor), so every parent precedes its children.
    Returns (parent [n] int32, node_token [n] int32, node_of [nc][P] int32)."""
    nc, P = tokens.shape
    index = {(): 0}
    parent, node_tok = [-1], [int(tokens[0, 0])]
    node_of = np.zeros((nc, P), np.int32)
    for c in range(nc):
        pre = ()
        for i in range(1, P):
            pre = pre + (int(tokens[c, i]),)
            if pre not in index:
                index[pre] = len(parent)
                parent.append(index[pre[:-1]])
                node_tok.append(int(tokens[c, i]))
            node_of[c, i] = index[pre]
    return np.array(parent, np.int32), np.array(node_tok, np.int32), node_of


def tree_round(cfg: Config, n: Optional[int] = None, rnd: int = 0, seed: int = 0, scale: float = math.sqrt(2.0)):
    """One round of token trees, one per sequence: the trie of cfg.nc candidate blocks whose drafts are
    Gumbel-max draws from prefix-keyed draft rows (``prefix_row``), padded to ``n`` nodes (default: the
    largest trie) with extra leaves whose tokens are drawn from their parent's draft row.

    Returns a dict: parent [nb][n], tokens [nb][n] (node 0 = the anchor), target_logits [nb][n][V]
    (row m: the target's row after node m's prefix), draft_logits [nb][n][V] (row m: the row node m's
    token was drawn from; row 0 zero), uniforms [nb][n] (entry 0 = r*), n, and the tries' sizes."""
    cand_zt, cand_zd, drafts, _ = prefix_keyed_round(cfg, rnd, seed, scale)
    anchor = anchors(cfg, rnd, seed)
    toks = block_tokens(anchor, drafts)
    tries = [trie_of(toks[b]) for b in range(cfg.nb)]
    sizes = [len(t[0]) for t in tries]
    n = max(sizes) if n is None else n
    assert n >= max(sizes)
    g = np.random.default_rng([cfg.cfg_id, seed, rnd, 91])
    parent = np.zeros((cfg.nb, n), np.int32)
    tokens = np.zeros((cfg.nb, n), np.int32)
    for b in range(cfg.nb):
        par, tok, _ = tries[b]
        par, tok = list(par), list(tok)
        while len(par) < n:                                   # padding leaves under random nodes
            par.append(int(g.integers(0, len(par))))
            tok.append(-1)
        parent[b], tokens[b] = par, tok
    zt = np.zeros((cfg.nb, n, cfg.vocab), np.float32)
    zd = np.zeros((cfg.nb, n, cfg.vocab), np.float32)
    for b in range(cfg.nb):
        pre = {0: ()}
        for m in range(1, n):
            p = int(parent[b, m])
            zd[b, m] = prefix_row(cfg, rnd, seed, 1, b, pre[p], scale)
            if tokens[b, m] < 0:                              # a padding leaf's token: a draw from its row
                gum = -np.log(-np.log(np.clip(g.random(cfg.vocab), 1e-300, 1.0 - 1e-16)))
                tokens[b, m] = int(np.argmax(zd[b, m].astype(np.float64) / cfg.temperature + gum))
            pre[m] = pre[p] + (int(tokens[b, m]),)
        for m in range(n):
            zt[b, m] = prefix_row(cfg, rnd, seed, 0, b, pre[m], scale)
    u = np.random.default_rng([cfg.cfg_id, seed, rnd, 92]).random((cfg.nb, n))
    return {"parent": parent, "tokens": tokens, "target_logits": zt, "draft_logits": zd, "uniforms": u, "n": n,
            "trie_sizes": sizes, "candidate_rows": (cand_zt, cand_zd)}


def random_tree(n: int, kind: str, rng: np.random.Generator) -> np.ndarray:
    """Parent array of a tree of n nodes: "chain", "star", "random" (each parent uniform over the
    earlier nodes) or "broom" (a chain of n // 2 nodes, the rest leaves of its last node)."""
    if kind == "chain":
        return np.array([-1] + list(range(n - 1)), np.int32)
    if kind == "star":
        return np.array([-1] + [0] * (n - 1), np.int32)
    if kind == "broom":
        h = max(1, n // 2)
        return np.array([-1] + list(range(h - 1)) + [h - 1] * (n - h), np.int32)
    return np.array([-1] + [int(rng.integers(0, m)) for m in range(1, n)], np.int32)


# ---------------------------------------------------------------- full layer stacks

@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """A striped stack: per layer "fir" (explicit long filter), "iir" (modal) or "attn"."""
    name: str
    cfg_id: int
    d: int
    heads: int
    head_dim: int
    kinds: Tuple[str, ...]
    taps_short: int
    taps_long: Tuple[int, ...]          # per layer, used by "fir" layers
    poles: int
    feature_layer: int
    feature_window: int
    kv_lens: Tuple[int, ...]            # committed length per sequence
    gamma: int
    nc: int = 1
    eps: float = 1e-6

    @property
    def nb(self) -> int:
        return len(self.kv_lens)

    @property
    def P(self) -> int:
        return self.gamma + 1

    @property
    def rows(self) -> int:
        return self.nb * self.nc * self.P


_STRIPE = ("fir", "fir", "iir", "attn")          # short-explicit, medium-regularised, long-implicit, attention
MODEL_CONFIGS: Dict[str, ModelConfig] = {
    "m4_small": ModelConfig("m4_small", 201, d=256, heads=2, head_dim=128, kinds=_STRIPE, taps_short=3,
                            taps_long=(7, 128, 0, 0), poles=16, feature_layer=2, feature_window=64,
                            kv_lens=(300, 37), gamma=6),
    "m4_long": ModelConfig("m4_long", 202, d=4096, heads=32, head_dim=128, kinds=_STRIPE, taps_short=3,
                           taps_long=(7, 128, 0, 0), poles=16, feature_layer=2, feature_window=64,
                           kv_lens=(262144,), gamma=12),
}


def model_scaled(mc: ModelConfig, **kw) -> ModelConfig:
    return dataclasses.replace(mc, **kw)


def _mgen(mc: ModelConfig, tag: int, seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000 + mc.cfg_id) * 1000 + tag) * 100003 + 17)
    return g


def make_model(mc: ModelConfig, seed: int = 0, device: str = "cpu") -> list:
    """Per layer: g [d] fp32 ~ 1 + N(0, 0.1^2); w_in [d][3d], w_out [d][d] bf16 ~ N(0, 1/d);
    w_short [Ts][3d] ~ N(0, 1/Ts); w_long [Tl][d] ~ N(0, 1/Tl); lam ~ U(0.5, 0.99); beta, c ~ N(0, 1/16)."""
    d, out = mc.d, []
    for l, kind in enumerate(mc.kinds):
        t = 100 * (l + 1)
        g = lambda k: _mgen(mc, t + k, seed, device)
        p = {"kind": kind,
             "g": 1.0 + 0.1 * torch.randn(d, generator=g(0), device=device),
             "w_in": (torch.randn((d, 3 * d), generator=g(1), device=device) * d ** -0.5).to(torch.bfloat16),
             "w_out": (torch.randn((d, d), generator=g(2), device=device) * d ** -0.5).to(torch.bfloat16)}
        if kind != "attn":
            Ts = mc.taps_short
            p["w_short"] = torch.randn((Ts, 3 * d), generator=g(3), device=device) * Ts ** -0.5
        if kind == "fir":
            Tl = mc.taps_long[l]
            p["w_long"] = torch.randn((Tl, d), generator=g(4), device=device) * Tl ** -0.5
        if kind == "iir":
            N = mc.poles
            p["lam"] = 0.5 + 0.49 * torch.rand((d, N), generator=g(5), device=device)
            p["beta"] = 0.25 * torch.randn((d, N), generator=g(6), device=device)
            p["c"] = 0.25 * torch.randn((d, N), generator=g(7), device=device)
        out.append(p)
    return out


def make_model_state(mc: ModelConfig, seed: int = 0, device: str = "cpu") -> dict:
    """Committed state: windows N(0,1), IIR N(0, 1/4), feature window and KV prefixes N(0,1) bf16.

    KV prefixes are [nb][H][L_b][Dh] per attention layer (a list per sequence)."""
    d, nb = mc.d, mc.nb
    layers = []
    for l, kind in enumerate(mc.kinds):
        t = 100 * (l + 1) + 50
        g = lambda k: _mgen(mc, t + k, seed, device)
        if kind == "attn":
            ks, vs = [], []
            for b, L in enumerate(mc.kv_lens):
                ks.append(torch.randn((mc.heads, L, mc.head_dim), generator=g(10 + 2 * b), device=device)
                          .to(torch.bfloat16))
                vs.append(torch.randn((mc.heads, L, mc.head_dim), generator=g(11 + 2 * b), device=device)
                          .to(torch.bfloat16))
            layers.append({"k": ks, "v": vs})
            continue
        st = {"short_win": torch.randn((nb, mc.taps_short - 1, 3 * d), generator=g(0), device=device)}
        if kind == "fir":
            st["long_win"] = torch.randn((nb, mc.taps_long[l] - 1, d), generator=g(1), device=device)
        else:
            st["iir"] = 0.5 * torch.randn((nb, d, mc.poles), generator=g(2), device=device)
        layers.append(st)
    feat = torch.randn((nb, mc.feature_window, d), generator=_mgen(mc, 99, seed, device), device=device)
    return {"layers": layers, "feature": feat.to(torch.bfloat16)}


def model_block_input(mc: ModelConfig, rnd: int = 0, seed: int = 0, device: str = "cpu") -> torch.Tensor:
    """x rows of the verified block [nb * nc * P][d] bf16 ~ N(0, 1); the candidates of a sequence share
    row 0 (the anchor)."""
    g = _mgen(mc, 900 + rnd, seed, device)
    x = torch.randn((mc.nb, mc.nc, mc.P, mc.d), generator=g, device=device)
    x[:, :, 0] = x[:, :1, 0]
    return x.to(torch.bfloat16).reshape(mc.rows, mc.d)


# ---------------------------------------------------------------- drafter

@dataclasses.dataclass(frozen=True)
class DrafterConfig:
    name: str
    cfg_id: int
    d_target: int
    d: int
    heads: int
    ffn: int
    vocab: int
    window: int
    layers: int = 2
    eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d // self.heads


DRAFTER_CONFIGS: Dict[str, DrafterConfig] = {
    # width 1024 over a W = 64 window of 4096-wide target states, two layers
    "d1k": DrafterConfig("d1k", 301, d_target=4096, d=1024, heads=8, ffn=4096, vocab=512, window=64),
    "d_small": DrafterConfig("d_small", 302, d_target=512, d=256, heads=2, ffn=512, vocab=512, window=64),
}


def make_drafter(dc: DrafterConfig, seed: int = 0, device: str = "cpu") -> dict:
    """Weights: projections bf16 ~ N(0, 1/fan_in); gains fp32 ~ 1 + N(0, 0.1^2); the tied embedding and
    the mask embedding bf16 ~ N(0, 1); the Markov bias fp32 ~ N(0, 1)."""
    g = lambda k: _mgen_d(dc, k, seed, device)
    bf = lambda shape, std, k: (torch.randn(shape, generator=g(k), device=device) * std).to(torch.bfloat16)
    d, F = dc.d, dc.ffn
    out = {"w_proj": bf((dc.d_target, d), dc.d_target ** -0.5, 1), "emb": bf((dc.vocab, d), 1.0, 2),
           "mask": bf((d,), 1.0, 3), "markov": torch.randn((dc.vocab, dc.vocab), generator=g(4), device=device),
           "g_f": 1.0 + 0.1 * torch.randn(d, generator=g(5), device=device), "layers": []}
    for l in range(dc.layers):
        k = 10 * (l + 1)
        out["layers"].append({"g1": 1.0 + 0.1 * torch.randn(d, generator=g(k), device=device),
                              "w_qkv": bf((d, 3 * d), d ** -0.5, k + 1), "w_o": bf((d, d), d ** -0.5, k + 2),
                              "g2": 1.0 + 0.1 * torch.randn(d, generator=g(k + 3), device=device),
                              "w_up": bf((d, F), d ** -0.5, k + 4), "w_down": bf((F, d), F ** -0.5, k + 5)})
    return out


def _mgen_d(dc: DrafterConfig, tag: int, seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1000 + dc.cfg_id) * 1000 + tag) * 100003 + 29)
    return g


def draft_round(dc: DrafterConfig, nb: int, gamma: int, rnd: int = 0, seed: int = 0, device: str = "cpu") -> dict:
    """A drafting round: window [nb][W][d_target] bf16 ~ N(0, 1), anchors, uniforms [nb][gamma] fp64."""
    g = _mgen_d(dc, 500 + rnd, seed, device)
    win = torch.randn((nb, dc.window, dc.d_target), generator=g, device=device).to(torch.bfloat16)
    gc = _mgen_d(dc, 600 + rnd, seed, "cpu")
    anchor = torch.randint(0, dc.vocab, (nb,), generator=gc, dtype=torch.int32)
    u = torch.rand((nb, gamma), generator=gc, dtype=torch.float64)
    return {"window": win, "anchor": anchor, "uniforms": u}
