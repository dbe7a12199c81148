"""GPU dense projection and RMS normalisation against the fp64 oracle.

Shapes span one and several 16-row tiles (ragged M), the block sizes of the
workloads (13 and 52 rows) against a 4096 x 12288 input projection, and K
and N from one tile up.  Tolerance: fp32 accumulation over K is bounded
elementwise by 2^-20 x (|x| |W|) (a loose multiple of K u for these K);
bf16 outputs add their half-ulp 2^-9 |y|, taken as 2^-8 |y|.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _packed(w):
    K, N = w.shape
    wp = torch.empty(hci.linear_packed_elems(K, N), dtype=torch.bfloat16, device="cuda")
    hci.linear_pack(w, wp)
    return wp


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


# every launch plan (strips x 16-row tiles per workgroup): 1 x 1 (64 x 1024: rows split to one
# tile per workgroup to fill the CUs), 2 x 1 (3 x 4112: two strips to fit one round of workgroups),
# 3 x 1 (13 x 12288), 4 x 1, 1 x 2, 2 x 2, 3 x 2, 4 x 2 (the short-K shapes), 1 x 4 (52 x 4096),
# 2 x 4 (76 x 3072), with ragged rows and strips
@pytest.mark.parametrize("M,K,N", [(1, 32, 16), (13, 4096, 12288), (52, 4096, 4096), (64, 1024, 1024),
                                   (76, 1024, 3072), (65, 64, 48), (200, 512, 256), (3, 96, 4112),
                                   (8, 64, 16384), (20, 64, 4096), (20, 64, 8192), (20, 64, 12288),
                                   (20, 64, 16384)])
@pytest.mark.parametrize("out_f32,with_res", [(False, False), (True, False), (False, True)])
def test_linear_matches_oracle(M, K, N, out_f32, with_res):
    say(f"linear M={M} K={K} N={N} out_f32={out_f32} residual={with_res}")
    x = synth.dense((M, K), 1.0, 1, device="cuda")
    w = synth.dense((K, N), K ** -0.5, 2, device="cuda")
    res = synth.dense((M, N), 1.0, 3, device="cuda") if with_res else None
    y = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    hci.linear(x, _packed(w), N, y, res)
    torch.cuda.synchronize()
    xh, wh = _f64(x), _f64(w)
    ref = oracle.linear(xh, wh, _f64(res) if with_res else None)
    bound = 2.0 ** -20 * (np.abs(xh) @ np.abs(wh)) + 1e-30
    if not out_f32:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(_f64(y) - ref)
    assert (err <= bound).all(), f"max err/bound {np.max(err / bound)}"


def test_linear_pack_layout():
    """Packed element [strip nt][tile kt][g][n][e] = W[32 kt + 8 g + e][16 nt + n] (the header's layout)."""
    K, N = 96, 48
    w = synth.dense((K, N), 1.0, 4, device="cuda")
    wp = _packed(w).view(torch.int16).cpu().numpy()
    wh = w.view(torch.int16).cpu().numpy()
    t = wp.reshape(N // 16, K // 32, 4, 16, 8)
    for nt in range(N // 16):
        for kt in range(K // 32):
            for g in range(4):
                np.testing.assert_array_equal(t[nt, kt, g], wh[32 * kt + 8 * g: 32 * kt + 8 * g + 8,
                                                             16 * nt: 16 * nt + 16].T)


@pytest.mark.parametrize("M,K", [(1, 64), (13, 4096), (52, 1000)])
def test_rmsnorm_matches_oracle(M, K):
    say(f"rmsnorm M={M} K={K}")
    x = synth.dense((M, K), 2.0, 5, device="cuda")
    g = synth.dense((K,), 1.0, 6, device="cuda").float()
    y = torch.empty_like(x)
    hci.rmsnorm(x, g, 1e-6, y)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(_f64(x), g.cpu().numpy(), 1e-6)
    err = np.abs(_f64(y) - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max()).all()
