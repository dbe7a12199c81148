"""The seeded input generator: determinism, shapes, distributions, planted agreement (CPU)."""
import numpy as np
import pytest

import oracle
from hybrid_conv_iir_amd import synth


def test_seeded_and_deterministic():
    cfg = synth.CONFIGS["tiny"]
    a, b = synth.make_layer(cfg), synth.make_layer(cfg)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    assert not np.array_equal(synth.make_layer(cfg, seed=1)["w_outer"], a["w_outer"])


def test_layer_distributions():
    cfg = synth.CONFIGS["mid8k"]
    p = synth.make_layer(cfg)
    assert p["w_outer"].shape == (128, 4096) and p["lam"].shape == (4096, 16)
    assert 0.5 <= p["lam"].min() and p["lam"].max() <= 0.99
    assert abs(p["beta"].var() - 1 / 16) < 0.003
    assert abs(p["w_outer"].var() - 1 / 128) < 0.0005


def test_bf16_rounding_is_nearest_even():
    import torch
    vals = torch.tensor([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=torch.float32)
    bits = synth.bf16_bits(vals)
    np.testing.assert_array_equal(oracle.as_f64(bits), [1.0, 1.0, 1.0 + 2 ** -6, -2.5])


def test_geometric_agreement_planted_length_is_the_greedy_k():
    cfg = synth.CONFIGS["long262k"]
    lens = []
    for rnd in range(40):
        drafts, zt, ln = synth.geometric_agreement(cfg, rnd)
        k, _, _ = oracle.greedy_accept(zt[0, 0], drafts[0, 0])
        assert k == ln[0, 0]
        lens.append(k)
    assert 0 < np.mean(lens) < cfg.gamma


def test_gumbel_drafts_follow_draft_distribution():
    cfg = synth.scaled(synth.CONFIGS["tiny"], vocab=4)
    z = np.array([[[[0.0, 1.0, -1.0, 0.5]]]], dtype=np.float32)
    counts = np.zeros(4)
    for rnd in range(4000):
        counts[synth.gumbel_drafts(cfg, z, rnd)[0, 0, 0]] += 1
    p = np.exp(z[0, 0, 0] - z.max())
    p /= p.sum()
    assert np.max(np.abs(counts / counts.sum() - p)) < 0.03


def test_kv_prefix_cpu_shape_and_moments():
    cfg = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(1000,), heads=2)
    k = synth.kv_prefix(cfg, 0, "k")
    assert tuple(k.shape) == (2, 1000, 128)
    kk = k.float().numpy()
    assert abs(kk.mean()) < 0.02 and abs(kk.std() - 1) < 0.02


def test_trie_of_candidates():
    """The trie of candidate blocks: one node per distinct prefix, parents before children, and every
    candidate position maps to the node whose path spells that candidate's prefix."""
    rng = np.random.default_rng(4)
    for _ in range(50):
        nc, P, V = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 4))
        toks = rng.integers(0, V, (nc, P)).astype(np.int32)
        toks[:, 0] = toks[0, 0]                                    # the shared anchor
        parent, node_tok, node_of = synth.trie_of(toks)
        assert parent[0] == -1 and all(0 <= parent[m] < m for m in range(1, len(parent)))
        prefixes = {tuple(toks[c, 1:i + 1]) for c in range(nc) for i in range(P)}
        assert len(parent) == len(prefixes)
        for c in range(nc):
            for i in range(P):
                m, spelled = int(node_of[c, i]), []
                while m != 0:
                    spelled.append(int(node_tok[m]))
                    m = int(parent[m])
                assert spelled[::-1] == list(toks[c, 1:i + 1])


def test_tree_round_shapes_and_rows():
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], vocab=4)
    tr = synth.tree_round(cfg)
    n = tr["n"]
    assert tr["parent"].shape == (cfg.nb, n) and tr["target_logits"].shape == (cfg.nb, n, cfg.vocab)
    assert max(tr["trie_sizes"]) == n and min(tr["trie_sizes"]) < cfg.nc * cfg.gamma + 1
    for b in range(cfg.nb):
        assert tr["parent"][b, 0] == -1 and all(0 <= tr["parent"][b, m] < m for m in range(1, n))
        assert ((tr["tokens"][b, 1:] >= 0) & (tr["tokens"][b, 1:] < cfg.vocab)).all()
