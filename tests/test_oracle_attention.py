"""Pins for the oracle's causal block attention (CPU only).

Pinned against torch's scaled_dot_product_attention in float64 with an
explicit mask, a pure-Python per-query loop on tiny shapes, and invariants:
an empty prefix gives o_0 = v_0, identical keys give the mean of the visible
values, and block rows after i never influence o_i.
"""
import math

import numpy as np
import pytest
import torch

from oracle import block_attention


def _case(seed, P=5, H=2, Dh=8, L=11, nblocks=2):
    r = np.random.default_rng(seed)
    q = r.standard_normal((P, H, Dh))
    k = r.standard_normal((P, H, Dh))
    v = r.standard_normal((P, H, Dh))
    cuts = np.linspace(0, L, nblocks + 1).astype(int)
    kp = r.standard_normal((H, L, Dh))
    vp = r.standard_normal((H, L, Dh))
    kb = [kp[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    vb = [vp[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    return q, k, v, kb, vb, kp, vp


def _sdpa_reference(q, k, v, kp, vp):
    P, H, Dh = q.shape
    L = kp.shape[1]
    keys = torch.from_numpy(np.concatenate([kp, k.transpose(1, 0, 2)], axis=1))    # [H][L+P][Dh]
    vals = torch.from_numpy(np.concatenate([vp, v.transpose(1, 0, 2)], axis=1))
    qq = torch.from_numpy(q.transpose(1, 0, 2).copy())                                # [H][P][Dh]
    mask = torch.ones((P, L + P), dtype=torch.bool)
    for i in range(P):
        mask[i, L + i + 1:] = False
    o = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask)
    return o.numpy().transpose(1, 0, 2)


def _matches_sdpa(attn, seed=0, **kw):
    q, k, v, kb, vb, kp, vp = _case(seed, **kw)
    got = attn(q, k, v, kb, vb)
    ref = _sdpa_reference(q, k, v, kp, vp)
    return np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("seed,P,L", [(0, 5, 11), (1, 13, 300), (2, 1, 7), (3, 7, 0)])
def test_attention_matches_sdpa_fp64(seed, P, L):
    assert _matches_sdpa(block_attention, seed=seed, P=P, L=L, nblocks=3 if L else 1)


def test_attention_pure_python_loop():
    q, k, v, kb, vb, kp, vp = _case(7, P=3, H=1, Dh=4, L=5, nblocks=1)
    got = block_attention(q, k, v, kb, vb)
    keys = [kp[0, j] for j in range(5)] + [k[j, 0] for j in range(3)]
    vals = [vp[0, j] for j in range(5)] + [v[j, 0] for j in range(3)]
    for i in range(3):
        n = 5 + i + 1
        sc = [sum(q[i, 0, e] * keys[j][e] for e in range(4)) / 2.0 for j in range(n)]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        tot = sum(w)
        ref = [sum(w[j] * vals[j][e] for j in range(n)) / tot for e in range(4)]
        np.testing.assert_allclose(got[i, 0], ref, rtol=1e-13, atol=1e-14)


def test_attention_empty_prefix_first_query_is_own_value():
    r = np.random.default_rng(8)
    q, k, v = (r.standard_normal((4, 3, 16)) for _ in range(3))
    empty = [np.zeros((3, 0, 16))]
    o = block_attention(q, k, v, empty, empty)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)


def test_attention_identical_keys_average_values():
    r = np.random.default_rng(9)
    P, H, Dh, L = 4, 2, 8, 6
    key = r.standard_normal(Dh)
    q = r.standard_normal((P, H, Dh))
    k = np.broadcast_to(key, (P, H, Dh)).copy()
    v = r.standard_normal((P, H, Dh))
    kp = np.broadcast_to(key, (H, L, Dh)).copy()
    vp = r.standard_normal((H, L, Dh))
    o = block_attention(q, k, v, [kp], [vp])
    for i in range(P):
        vis = np.concatenate([vp, v[: i + 1].transpose(1, 0, 2)], axis=1)
        np.testing.assert_allclose(o[i], vis.mean(axis=1), rtol=1e-12, atol=1e-14)


def test_attention_future_block_rows_do_not_leak():
    q, k, v, kb, vb, _, _ = _case(10, P=6, L=9)
    base = block_attention(q, k, v, kb, vb)
    for j in range(1, 6):
        k2, v2 = k.copy(), v.copy()
        k2[j] += 5.0
        v2[j] -= 3.0
        o2 = block_attention(q, k2, v2, kb, vb)
        np.testing.assert_array_equal(o2[:j], base[:j])
        assert np.max(np.abs(o2[j:] - base[j:])) > 1e-3


def test_attention_pin_catches_missing_mask_and_scale():
    def unmasked(q, k, v, kb, vb):       # planted mistake: block keys after i visible
        P = q.shape[0]
        out = np.zeros(q.shape)
        for i in range(P):
            out[i] = block_attention(q[i:i + 1], k[[i]], v[[i]], kb + [k.transpose(1, 0, 2)],
                                     vb + [v.transpose(1, 0, 2)])[0]
        return out

    def unscaled(q, k, v, kb, vb):       # planted mistake: no 1/sqrt(Dh)
        s = math.sqrt(q.shape[2])
        return block_attention(q * s, k, v, kb, vb)
    assert not _matches_sdpa(unmasked, seed=11)
    assert not _matches_sdpa(unscaled, seed=11)
