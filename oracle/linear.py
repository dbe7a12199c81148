"""Oracle: dense projections and RMS normalisation around the mixers (fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The full hybrid layers (EvSpark digest, Figure 1(a): a StripedHyena2 target)
put dense input and output projections and a normalisation around each
mixer; the pages give no equations for them, so the plain definitions are
used: y = x W (+ residual) and RMSNorm(x) = x * g / sqrt(mean(x^2) + eps).
"""
from __future__ import annotations

import numpy as np

from .layer import as_f64


def linear(x, w, residual=None) -> np.ndarray:
    """y [M][N] = x [M][K] @ w [K][N] (+ residual), fp64 (numpy matmul as the product primitive)."""
    y = as_f64(x) @ as_f64(w)
    if residual is not None:
        y = y + as_f64(residual)
    return y


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """Each row divided by the root of its mean square (plus eps), times the per-channel gain."""
    xx = as_f64(x)
    ms = np.mean(xx * xx, axis=-1, keepdims=True)
    return xx / np.sqrt(ms + eps) * as_f64(gamma)
