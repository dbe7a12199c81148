"""hci_verify_block_noalloc (the library's own scratch array as the verify
workspace) gives the same outputs as hci_verify_block with a caller-allocated
workspace, bit for bit, on two calls in a row -- the second with a smaller
input, so it runs over what the first left in the array -- and rejects sizes
beyond the array before enqueueing anything.  Runs alone in a fresh process
and after the other GPU tests (the array persists across calls)."""
import numpy as np
import pytest
import torch

from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import Case, say

pytestmark = pytest.mark.gpu

_OUTS = ("f", "s", "y", "o")


def _compare(case: Case, label: str):
    cfg = case.cfg
    ref = dv.DeviceBlock(case.lay, cfg.nb, cfg.nc, cfg.gamma)
    ref.set_inputs(case.blk.x, case.blk.q, case.blk.k, case.blk.v)
    say(f"noalloc {label}: {cfg.name} nb={cfg.nb} nc={cfg.nc} gamma={cfg.gamma} L={cfg.kv_lens}")
    need = hci.verify_workspace_bytes(case.lay.c, cfg.nb, cfg.nc, cfg.gamma, cfg.max_kv_len)
    assert 0 < need <= hci.NOALLOC_SCRATCH_BYTES
    for t in _OUTS:                                # the outputs must come from the call under test
        getattr(case.blk, t).fill_(float("nan"))
    hci.verify_block_noalloc(case.lay.c, case.st.c, case.blk.c, cfg.nb, cfg.nc, cfg.gamma, cfg.max_kv_len)
    dv.verify(case.lay, case.st, ref, cfg.max_kv_len)
    torch.cuda.synchronize()
    for t in _OUTS:
        got, want = dv.to_host(getattr(case.blk, t)), dv.to_host(getattr(ref, t))
        np.testing.assert_array_equal(got.view(np.uint8), want.view(np.uint8), err_msg=f"{label} {t}")
    assert [int(v) for v in dv.to_host(case.st.status)] == [0] * cfg.nb


def test_noalloc_matches_workspace_verify_two_calls():
    big = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(8192, 3001), mode="greedy")
    small = synth.scaled(synth.CONFIGS["mid8k"], d=512, heads=4, kv_lens=(1000,), gamma=6, mode="greedy")
    _compare(Case(big, host_prefix=False), "first call")
    _compare(Case(small, host_prefix=False), "second call, smaller")


def test_noalloc_fp32_layer_and_empty_prefix():
    tiny = synth.CONFIGS["tiny"]
    _compare(Case(tiny, host_prefix=False), "fp32")
    _compare(Case(synth.scaled(tiny, kv_lens=(0,)), host_prefix=False), "fp32, empty prefix")


def test_noalloc_long_context_fits():
    """The long-context workload (262144-token prefix, 32 x 128 heads, gamma 12) runs in the array."""
    cfg = synth.CONFIGS["long262k"]
    _compare(Case(cfg, host_prefix=False), "long context")


def test_noalloc_rejects_sizes_beyond_the_array():
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], kv_lens=(0, 0, 0, 0))
    case = Case(cfg, host_prefix=False)
    big_len = 65536
    need = hci.verify_workspace_bytes(case.lay.c, cfg.nb, cfg.nc, cfg.gamma, big_len)
    assert need > hci.NOALLOC_SCRATCH_BYTES
    st = dv.DeviceState(case.lay, cfg.nb, big_len + 64)
    say("noalloc: a size beyond the array is rejected on the host")
    with pytest.raises(hci.HciError) as e:
        hci.verify_block_noalloc(case.lay.c, st.c, case.blk.c, cfg.nb, cfg.nc, cfg.gamma, big_len)
    assert e.value.status == hci.EWORKSPACE
