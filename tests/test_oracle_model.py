"""Pins for the oracle's hybrid layer stack (CPU only).

* block forward + slice at k equals k+1 one-row steps, for every k (the
  replay definition of the state contract), with rounding off;
* streaming: several blocks with slices in between equal one block over the
  whole sequence from the empty state (zero windows and IIR state, no KV) --
  brute force over the full history, which checks every window, state and
  cache hand-over;
* bf16 rounding equals torch's float32 -> bfloat16 conversion.
The layer equations themselves (gating order, projection split) are a
reading of the pages, which print none: parity unpinned beyond these checks.
"""
import numpy as np
import pytest
import torch

from oracle import model as M


def _model(r, d=8, H=2, kinds=("fir", "iir", "attn", "fir"), Ts=3, Tl=(5, 0, 0, 2), N=4, W=6, feature_layer=1):
    mixers = []
    for i, kind in enumerate(kinds):
        mx = M.Mixer(kind=kind, g=1.0 + 0.1 * r.standard_normal(d), w_in=r.standard_normal((d, 3 * d)) / np.sqrt(d),
                     w_out=r.standard_normal((d, d)) / np.sqrt(d))
        if kind != "attn":
            mx.w_short = r.standard_normal((Ts, 3 * d)) / np.sqrt(Ts)
        if kind == "fir":
            mx.w_long = r.standard_normal((Tl[i], d)) / np.sqrt(Tl[i])
        if kind == "iir":
            mx.lam = r.uniform(0.5, 0.99, (d, N))
            mx.beta = r.normal(0, 0.25, (d, N))
            mx.c = r.normal(0, 0.25, (d, N))
        mixers.append(mx)
    return M.Model(mixers, d, H, d // H, 1e-6, feature_layer, W)


def _state(model, r, L=3, zero=False):
    d, H, Dh = model.d, model.heads, model.head_dim
    f = (lambda s: np.zeros(s)) if zero else (lambda s: r.standard_normal(s))
    layers = []
    for mx in model.mixers:
        if mx.kind == "attn":
            layers.append(M.LayerState(k_blocks=[f((H, 0 if zero else L, Dh))], v_blocks=[f((H, 0 if zero else L, Dh))]))
            continue
        ls = M.LayerState(short_win=f((mx.w_short.shape[0] - 1, 3 * d)))
        if mx.kind == "fir":
            ls.long_win = f((mx.w_long.shape[0] - 1, d))
        else:
            ls.iir = f((d, mx.lam.shape[1])) * 0.5
        layers.append(ls)
    return M.ModelState(layers, f((model.feature_window, d)))


def _cat(blocks):
    return np.concatenate(blocks, axis=1)


def _same_state(a, b, tol):
    for la, lb in zip(a.layers, b.layers):
        for name in ("short_win", "long_win", "iir"):
            x, y = getattr(la, name), getattr(lb, name)
            assert (x is None) == (y is None)
            if x is not None:
                np.testing.assert_allclose(x, y, rtol=0, atol=tol)
        if la.k_blocks:
            np.testing.assert_allclose(_cat(la.k_blocks), _cat(lb.k_blocks), atol=tol)
            np.testing.assert_allclose(_cat(la.v_blocks), _cat(lb.v_blocks), atol=tol)
    np.testing.assert_allclose(a.feature, b.feature, atol=tol)


@pytest.mark.parametrize("seed", [0, 1])
def test_block_plus_slice_equals_sequential_steps(seed):
    r = np.random.default_rng(seed)
    model = _model(r)
    st = _state(model, r)
    P = 7
    x = r.standard_normal((P, model.d))
    fwd = M.model_verify_block(model, st, x, rounding=False)
    for k in range(P):
        blk = M.model_slice_state(model, st, fwd, k)
        seq, outs = M.model_sequential_steps(model, st, x, k + 1, rounding=False)
        _same_state(blk, seq, 1e-12)
        np.testing.assert_allclose(fwd["x"][-1][: k + 1], outs, atol=1e-12)


def test_streaming_equals_one_block_from_the_empty_state():
    """Blocks of 3, 1, 5 and 4 rows with slices in between = one 13-row block from zero state."""
    r = np.random.default_rng(5)
    model = _model(r, kinds=("iir", "fir", "attn", "fir", "attn"), Tl=(0, 6, 0, 3, 0), W=20)
    st0 = _state(model, r, zero=True)
    x = r.standard_normal((13, model.d))
    whole = M.model_verify_block(model, st0, x, rounding=False)
    st, outs, i = st0, [], 0
    for n in (3, 1, 5, 4):
        fwd = M.model_verify_block(model, st, x[i: i + n], rounding=False)
        outs.append(fwd["x"][-1])
        st = M.model_slice_state(model, st, fwd, n - 1)
        i += n
    np.testing.assert_allclose(np.concatenate(outs), whole["x"][-1], atol=1e-10)
    np.testing.assert_allclose(st.feature[-13:], whole["x"][model.feature_layer + 1], atol=1e-10)
    final = M.model_slice_state(model, st0, whole, 12)
    _same_state(st, final, 1e-10)


def test_bf16_round_matches_torch():
    r = np.random.default_rng(9)
    v = (r.standard_normal(20000) * np.exp(r.uniform(-20, 20, 20000))).astype(np.float32)
    v[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]      # ties on both sides, zero
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(M.bf16_round(v.astype(np.float64)), ref)
