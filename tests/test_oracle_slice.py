"""Pins for the oracle's slicing and the block-forward / state-restoration contract (CPU only).

* EvSpark Figure 1(d) worked example (tests/golden/fig1_worked_example.json):
  with gamma = 6 and three accepted drafts the KV prefix grows by 4, the
  outer window keeps u2 and u3, and the IIR state is s3.
* For every k, one block forward plus a slice at k equals k+1 sequential
  single-position steps (the replay the method avoids): windows, IIR state
  and KV rows bit for bit, outputs to rounding.
* A planted mistake (keeping s_{k+1}) is caught by the contract.
* Sequence level (greedy): a speculative decode loop with a toy fp64 LM head
  emits exactly the tokens of plain sequential greedy decoding.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import Layer, SeqState, block_attention, sequential_steps, slice_state, verify_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer(r, d, Ts, To, N):
    return Layer(r.normal(0, 1 / np.sqrt(Ts), (Ts, d)), r.normal(0, 1 / np.sqrt(To), (To, d)),
                 r.uniform(0.5, 0.99, (d, N)), r.normal(0, 0.25, (d, N)), r.normal(0, 0.25, (d, N)))


def _state(r, d, Ts, To, N, H, Dh, L):
    return SeqState(r.standard_normal((Ts - 1, d)), r.standard_normal((To - 1, d)),
                    r.standard_normal((d, N)) * 0.5,
                    [r.standard_normal((H, L, Dh))], [r.standard_normal((H, L, Dh))])


def _block(r, P, d, H, Dh):
    return (r.standard_normal((P, d)), r.standard_normal((P, H, Dh)),
            r.standard_normal((P, H, Dh)), r.standard_normal((P, H, Dh)))


def _kv(st):
    return (np.concatenate([oracle.as_f64(b) for b in st.k_blocks], axis=1),
            np.concatenate([oracle.as_f64(b) for b in st.v_blocks], axis=1))


def test_fig1d_worked_example():
    with open(os.path.join(GOLDEN, "fig1_worked_example.json")) as fh:
        fx = json.load(fh)
    r = np.random.default_rng(3)
    gamma, k = fx["gamma"], fx["state_index"]
    d, Ts, To, N, H, Dh, L = 8, 3, fx["outer_taps_implied"], 4, 2, 8, 10
    lay = _layer(r, d, Ts, To, N)
    st = _state(r, d, Ts, To, N, H, Dh, L)
    x, q, kk, vv = _block(r, gamma + 1, d, H, Dh)
    fwd = verify_block(lay, st, x, q, kk, vv)
    new = slice_state(st, x, fwd, kk, vv, k)
    assert new.kv_len - st.kv_len == fx["kv_growth"]
    pos = fx["outer_window_positions"]
    np.testing.assert_array_equal(new.outer_win, fwd["f"][pos])        # u2, u3
    np.testing.assert_array_equal(new.short_win, x[pos])               # x2, x3
    np.testing.assert_array_equal(new.iir, fwd["s"][fx["iir_state_index"]])
    kn, vn = _kv(new)
    np.testing.assert_array_equal(kn[:, L:], kk[: k + 1].transpose(1, 0, 2))
    np.testing.assert_array_equal(vn[:, L:], vv[: k + 1].transpose(1, 0, 2))


def _contract_holds(slicer, gamma=6, Ts=3, To=7, seed=0):
    r = np.random.default_rng(seed)
    d, N, H, Dh, L = 6, 16, 2, 8, 20
    lay = _layer(r, d, Ts, To, N)
    st = _state(r, d, Ts, To, N, H, Dh, L)
    x, q, kk, vv = _block(r, gamma + 1, d, H, Dh)
    fwd = verify_block(lay, st, x, q, kk, vv)
    for k in range(gamma + 1):
        blk = slicer(st, x, fwd, kk, vv, k)
        seq, outs = sequential_steps(lay, st, x, q, kk, vv, k + 1)
        same = (np.array_equal(blk.short_win, seq.short_win) and np.array_equal(blk.outer_win, seq.outer_win)
                and np.array_equal(blk.iir, seq.iir) and blk.kv_len == seq.kv_len
                and all(np.array_equal(a, b) for a, b in zip(_kv(blk), _kv(seq)))
                and np.array_equal(fwd["f"][: k + 1], outs["f"]) and np.array_equal(fwd["s"][: k + 1], outs["s"])
                and np.array_equal(fwd["y"][: k + 1], outs["y"])
                and np.max(np.abs(fwd["o"][: k + 1] - outs["o"])) <= 1e-12)
        if not same:
            return False
    return True


@pytest.mark.parametrize("gamma,Ts,To", [(6, 3, 7), (12, 3, 7), (6, 3, 3), (3, 1, 2), (12, 4, 20)])
def test_block_plus_slice_equals_sequential_steps(gamma, Ts, To):
    assert _contract_holds(slice_state, gamma=gamma, Ts=Ts, To=To, seed=gamma + To)


def test_contract_catches_off_by_one_state():
    def keeps_next(st, x, fwd, kb, vb, k):     # planted mistake: s_{k+1} kept
        new = slice_state(st, x, fwd, kb, vb, k)
        new.iir = np.array(fwd["s"][min(k + 1, len(fwd["s"]) - 1)])
        return new
    assert not _contract_holds(keeps_next)


def test_contract_catches_stale_window():
    def stale(st, x, fwd, kb, vb, k):          # planted mistake: outer window one position short
        good = slice_state(st, x, fwd, kb, vb, k)
        short = slice_state(st, x, fwd, kb, vb, max(k - 1, 0))
        return SeqState(good.short_win, short.outer_win, good.iir, good.k_blocks, good.v_blocks)
    assert not _contract_holds(stale)


def test_sequence_level_greedy_exactness():
    """A toy fp64 LM head turns the layer's outputs into logits; speculative rounds emit the
    same tokens as sequential greedy decoding (EvSpark digest, Interpretation: sequence-level
    exactness).  Parity of this toy head with the EvSpark target is unpinned; the equality of
    the two decoding procedures is what is checked."""
    r = np.random.default_rng(21)
    d, Ts, To, N, H, Dh, V = 8, 3, 5, 4, 2, 4, 8
    lay = _layer(r, d, Ts, To, N)
    E_x, E_q, E_k, E_v = (r.standard_normal((V, d)), r.standard_normal((V, H, Dh)),
                          r.standard_normal((V, H, Dh)), r.standard_normal((V, H, Dh)))
    W_head = r.standard_normal((V, d + H * Dh))

    def logits(fwd, i):
        feat = np.concatenate([fwd["y"][i], fwd["o"][i].reshape(-1)])
        return W_head @ feat

    st0 = _state(r, d, Ts, To, N, H, Dh, 6)
    n_tokens = 40
    # sequential greedy decoding
    st, tok, seq_out = st0, 3, []
    for _ in range(n_tokens):
        fwd = verify_block(lay, st, E_x[[tok]], E_q[[tok]], E_k[[tok]], E_v[[tok]])
        st = slice_state(st, E_x[[tok]], fwd, E_k[[tok]], E_v[[tok]], 0)
        tok = int(np.argmax(logits(fwd, 0)))
        seq_out.append(tok)
    # speculative decoding: random drafts, some of which happen to be right
    st, anchor, spec_out, gamma = st0, 3, [], 4
    drafts_rng = np.random.default_rng(5)
    while len(spec_out) < n_tokens:
        guess = [seq_out[len(spec_out) + j] if drafts_rng.random() < 0.6 and len(spec_out) + j < n_tokens
                 else int(drafts_rng.integers(0, V)) for j in range(gamma)]
        toks = np.array([anchor] + guess)
        fwd = verify_block(lay, st, E_x[toks], E_q[toks], E_k[toks], E_v[toks])
        zt = np.stack([logits(fwd, i) for i in range(gamma + 1)])
        k, nxt, _ = oracle.greedy_accept(zt, np.array(guess))
        st = slice_state(st, E_x[toks], fwd, E_k[toks], E_v[toks], k)
        spec_out.extend(guess[:k] + [nxt])
        anchor = nxt
    assert spec_out[:n_tokens] == seq_out
