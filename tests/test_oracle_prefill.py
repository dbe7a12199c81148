"""Pins for the oracle's prefill (CPU only): it equals T sequential single-position
steps (the replay definition), the numpy.convolve FIR equals the plain FIR, and the
final-state IIR scan equals the state-keeping scan."""
import numpy as np
import pytest

import oracle
from oracle import Layer, SeqState


def _setup(seed, d=6, Ts=3, To=7, N=16, H=2, Dh=8, L=5, T=40):
    r = np.random.default_rng(seed)
    lay = Layer(r.normal(0, 1 / np.sqrt(Ts), (Ts, d)), r.normal(0, 1 / np.sqrt(To), (To, d)),
                r.uniform(0.5, 0.99, (d, N)), r.normal(0, 0.25, (d, N)), r.normal(0, 0.25, (d, N)))
    st = SeqState(r.standard_normal((Ts - 1, d)), r.standard_normal((To - 1, d)), r.standard_normal((d, N)) * 0.5,
                  [r.standard_normal((H, L, Dh))], [r.standard_normal((H, L, Dh))])
    x = r.standard_normal((T, d))
    k = r.standard_normal((T, H, Dh))
    v = r.standard_normal((T, H, Dh))
    q = r.standard_normal((T, H, Dh))
    return lay, st, x, q, k, v


@pytest.mark.parametrize("T,To", [(1, 7), (3, 7), (40, 7), (40, 128), (200, 3)])
def test_prefill_equals_sequential_steps(T, To):
    lay, st, x, q, k, v = _setup(T + To, To=To, T=T)
    new, y = oracle.prefill_state(lay, st, x, k, v)
    seq, outs = oracle.sequential_steps(lay, st, x, q, k, v, T)
    np.testing.assert_array_equal(new.short_win, seq.short_win)
    np.testing.assert_array_equal(new.outer_win, seq.outer_win)
    np.testing.assert_array_equal(new.iir, seq.iir)
    np.testing.assert_array_equal(y, outs["y"])
    assert new.kv_len == seq.kv_len
    for a, b in zip(new.k_blocks, seq.k_blocks[:1] + [np.concatenate(seq.k_blocks[1:], axis=1)]):
        np.testing.assert_array_equal(a, b)


def test_long_fir_equals_plain_fir():
    r = np.random.default_rng(3)
    for T, taps in ((1, 128), (50, 3), (300, 128), (7, 1)):
        blk, win, w = r.standard_normal((T, 5)), r.standard_normal((taps - 1, 5)), r.standard_normal((taps, 5))
        np.testing.assert_allclose(oracle.depthwise_fir_long(blk, win, w), oracle.depthwise_fir(blk, win, w),
                                   rtol=1e-12, atol=1e-12)


def test_iir_scan_equals_state_keeping_scan():
    r = np.random.default_rng(4)
    g, s0 = r.standard_normal((60, 4)), r.standard_normal((4, 16))
    lam, beta, c = r.uniform(0.5, 0.99, (4, 16)), r.normal(0, 0.25, (4, 16)), r.normal(0, 0.25, (4, 16))
    s_last, y = oracle.iir_scan(g, s0, lam, beta, c)
    S, Y = oracle.modal_iir(g, s0, lam, beta, c)
    np.testing.assert_array_equal(s_last, S[-1])
    np.testing.assert_array_equal(y, Y)


def test_prefill_split_composes():
    """prefill(T) == prefill(T1) then prefill(T - T1), the property the GPU long-prompt test uses."""
    lay, st, x, q, k, v = _setup(9, To=20, T=90)
    full, y = oracle.prefill_state(lay, st, x, k, v)
    a, y1 = oracle.prefill_state(lay, st, x[:37], k[:37], v[:37])
    b, y2 = oracle.prefill_state(lay, a, x[37:], k[37:], v[37:])
    np.testing.assert_allclose(b.iir, full.iir, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b.outer_win, full.outer_win, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-13)
