"""Pins for the oracle's depthwise FIRs and modal IIR (CPU only).

The FIRs are pinned by brute-force full convolution from zero state and by
delta taps; the IIR by its closed form (convolution with the materialised
impulse response plus the decayed initial state), by scipy's one-pole
``lfilter`` and by the lambda = 0 and beta = 0 special cases.  Each pin is
also run against a planted mistake to show it would catch it.
"""
import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import depthwise_fir, modal_iir



def _rng(seed):
    return np.random.default_rng(seed)


def _blockwise_fir(fir, hist, taps, P):
    """Run ``fir`` over a zero-started history in blocks of P, windows taken from the history."""
    T, d = taps.shape
    W = T - 1
    padded = np.concatenate([np.zeros((W, d)), hist], axis=0)
    out = []
    for start in range(0, hist.shape[0], P):
        blk = hist[start:start + P]
        win = padded[start:start + W]            # the W inputs before the block
        out.append(fir(blk, win, taps))
    return np.concatenate(out, axis=0)


def _fir_matches_convolution(fir, T=7, d=5, n=41, P=6, seed=0):
    r = _rng(seed)
    hist = r.standard_normal((n, d))
    taps = r.standard_normal((T, d))
    got = _blockwise_fir(fir, hist, taps, P)
    ref = np.stack([np.convolve(hist[:, ch], taps[:, ch])[:n] for ch in range(d)], axis=1)
    return np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("T,P", [(3, 7), (7, 7), (7, 3), (128, 13), (1, 4)])
def test_fir_equals_full_convolution(T, P):
    assert _fir_matches_convolution(depthwise_fir, T=T, P=P, n=3 * P + 2)


def test_fir_delta_taps_shift():
    r = _rng(1)
    d, T, P = 4, 7, 7
    win = r.standard_normal((T - 1, d))
    blk = r.standard_normal((P, d))
    full = np.concatenate([win, blk])
    for lag in range(T):
        taps = np.zeros((T, d))
        taps[lag] = 1.0
        out = depthwise_fir(blk, win, taps)
        np.testing.assert_array_equal(out, full[T - 1 - lag: T - 1 - lag + P])


def test_fir_identity_taps():
    r = _rng(2)
    x = r.standard_normal((7, 3))
    out = depthwise_fir(x, r.standard_normal((2, 3)), np.array([[1.0] * 3, [0.0] * 3, [0.0] * 3]))
    np.testing.assert_array_equal(out, x)


def test_fir_pin_catches_correlation():
    def correlated(blk, win, taps):          # planted mistake: taps reversed (correlation)
        return depthwise_fir(blk, win, taps[::-1])
    assert not _fir_matches_convolution(correlated)


# ------------------------------------------------------------------ IIR

def _params(r, d, N):
    lam = r.uniform(0.5, 0.99, (d, N))
    beta = r.normal(0, 0.25, (d, N))
    c = r.normal(0, 0.25, (d, N))
    return lam, beta, c


def _iir_closed_form(g, s0, lam, beta, c):
    """y_i = sum_{t<=i} h[i-t] g_t + sum_n c lam^(i+1) s0 with h[t] = sum_n c lam^t beta."""
    T, d = g.shape
    t = np.arange(T)
    y = np.zeros((T, d))
    for ch in range(d):
        h = (c[ch][None, :] * lam[ch][None, :] ** t[:, None] * beta[ch][None, :]).sum(axis=1)
        y[:, ch] = np.convolve(g[:, ch], h)[:T]
        y[:, ch] += (c[ch][None, :] * lam[ch][None, :] ** (t[:, None] + 1) * s0[ch][None, :]).sum(axis=1)
    return y


def _iir_matches_closed_form(iir, T=4096, d=3, N=16, seed=3, zero_state=False, blocks=13):
    r = _rng(seed)
    lam, beta, c = _params(r, d, N)
    g = r.standard_normal((T, d))
    s0 = np.zeros((d, N)) if zero_state else r.standard_normal((d, N))
    ys = []
    s = s0
    for start in range(0, T, blocks):
        S, Y = iir(g[start:start + blocks], s, lam, beta, c)
        ys.append(Y)
        s = S[-1]
    got = np.concatenate(ys)
    ref = _iir_closed_form(g, s0, lam, beta, c)
    return np.max(np.abs(got - ref)) <= 1e-11 * np.max(np.abs(ref))


def test_iir_closed_form_zero_state():
    assert _iir_matches_closed_form(modal_iir, zero_state=True)


def test_iir_closed_form_with_state():
    assert _iir_matches_closed_form(modal_iir, zero_state=False, T=600)


def test_iir_kept_states_closed_form():
    r = _rng(4)
    d, N, P = 2, 16, 13
    lam, beta, c = _params(r, d, N)
    g = r.standard_normal((P, d))
    s0 = r.standard_normal((d, N))
    S, _ = modal_iir(g, s0, lam, beta, c)
    for i in range(P):
        ref = lam ** (i + 1) * s0 + sum(lam ** (i - t) * beta * g[t][:, None] for t in range(i + 1))
        np.testing.assert_allclose(S[i], ref, rtol=1e-13, atol=1e-14)


def test_iir_one_pole_is_lfilter():
    r = _rng(5)
    d, T = 3, 500
    lam, beta, c = _params(r, d, 1)
    g = r.standard_normal((T, d))
    _, Y = modal_iir(g, np.zeros((d, 1)), lam, beta, c)
    for ch in range(d):
        ref = scipy.signal.lfilter([beta[ch, 0] * c[ch, 0]], [1.0, -lam[ch, 0]], g[:, ch])
        np.testing.assert_allclose(Y[:, ch], ref, rtol=1e-12, atol=1e-13)


def test_iir_lambda_zero_is_one_tap():
    r = _rng(6)
    d, N, P = 4, 16, 9
    _, beta, c = _params(r, d, N)
    g = r.standard_normal((P, d))
    _, Y = modal_iir(g, r.standard_normal((d, N)), np.zeros((d, N)), beta, c)
    np.testing.assert_allclose(Y, g * (c * beta).sum(axis=1)[None, :], rtol=1e-13, atol=1e-15)


def test_iir_beta_zero_pure_decay():
    r = _rng(7)
    d, N, P = 4, 16, 9
    lam, _, c = _params(r, d, N)
    s0 = r.standard_normal((d, N))
    _, Y = modal_iir(r.standard_normal((P, d)), s0, lam, np.zeros((d, N)), c)
    for i in range(P):
        np.testing.assert_allclose(Y[i], (c * lam ** (i + 1) * s0).sum(axis=1), rtol=1e-13, atol=1e-15)


def test_iir_pin_catches_readout_before_update():
    def early_readout(g, s_prev, lam, beta, c):   # planted mistake: y read from s_{i-1}
        S, _ = modal_iir(g, s_prev, lam, beta, c)
        prev = np.concatenate([np.asarray(s_prev)[None], S[:-1]], axis=0)
        return S, (np.asarray(c)[None] * prev).sum(axis=2)
    assert not _iir_matches_closed_form(early_readout, T=200)


def test_iir_pin_catches_dropped_input_gain():
    def no_beta(g, s_prev, lam, beta, c):          # planted mistake: beta dropped
        return modal_iir(g, s_prev, lam, np.ones_like(beta), c)
    assert not _iir_matches_closed_form(no_beta, T=200)


def test_as_f64_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3E80, 0x7F7F], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.as_f64(bits), [1.0, -2.0, 0.0, 0.25, 3.3895313892515355e38])
