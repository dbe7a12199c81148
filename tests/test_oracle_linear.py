"""Pins for the oracle's projection and normalisation (CPU only)."""
import numpy as np

import oracle


def test_linear_equals_triple_loop():
    r = np.random.default_rng(0)
    x = r.standard_normal((3, 5))
    w = r.standard_normal((5, 4))
    res = r.standard_normal((3, 4))
    y = oracle.linear(x, w, res)
    for i in range(3):
        for j in range(4):
            acc = res[i, j]
            for k in range(5):
                acc += x[i, k] * w[k, j]
            assert abs(y[i, j] - acc) < 1e-12


def test_linear_permutation_and_identity():
    r = np.random.default_rng(1)
    x = r.standard_normal((7, 32))
    perm = r.permutation(32)
    P = np.eye(32)[:, perm]                  # column j of P picks input perm[j]
    np.testing.assert_array_equal(oracle.linear(x, P), x[:, perm])
    np.testing.assert_array_equal(oracle.linear(x, np.eye(32)), x)


def test_rmsnorm_unit_rms_and_scale_invariance():
    r = np.random.default_rng(2)
    x = r.standard_normal((4, 64)) * 3.0
    y = oracle.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(5.0 * x, np.ones(64), 0.0), y, rtol=1e-12)
    g = r.standard_normal(64)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 0.0), y * g, rtol=1e-12)
    # eps: a zero row stays zero instead of dividing by zero
    assert np.all(oracle.rmsnorm(np.zeros((1, 8)), np.ones(8), 1e-6) == 0.0)
