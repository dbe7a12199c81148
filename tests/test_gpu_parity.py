"""GPU parity: verify -> accept -> slice through the C ABI against the fp64 oracle.

Sizes span several KV tiles and a ragged tail; the long-context and
multi-candidate workloads run at their full sizes in the launch
configuration the benchmark times.  Tolerances: tests/gpu_harness.py.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import Case, assert_f32_close, assert_out_close, f64, say

pytestmark = pytest.mark.gpu

MARGIN = 1e-12


def _check_round(case: Case, heads=None, check_accept=True):
    cfg = case.cfg
    say(f"{cfg.name} nb={cfg.nb} nc={cfg.nc} gamma={cfg.gamma} L={cfg.kv_lens} verify+accept+slice")
    case.run_verify()
    case.run_accept()
    torch.cuda.synchronize()
    f = dv.to_host(case.blk.f)
    s = dv.to_host(case.blk.s)
    y = dv.to_host(case.blk.y)
    o = dv.to_host(case.blk.o)
    n_acc, nxt, best, marg = (dv.to_host(t) for t in (case.acc.n_acc, case.acc.next, case.acc.best, case.acc.margin))
    r_acc, r_next, r_best, r_marg = case.oracle_accept()
    if check_accept:
        assert (r_marg > MARGIN).all(), f"near-tie decision in the oracle: {r_marg.min()}"
        np.testing.assert_array_equal(n_acc, r_acc)
        np.testing.assert_array_equal(nxt, r_next)
        np.testing.assert_array_equal(best, r_best)
        if cfg.mode == "greedy":
            np.testing.assert_array_equal(marg, r_marg)
        else:
            np.testing.assert_allclose(marg, r_marg, rtol=1e-6, atol=1e-15)
        if case.ri["planted_len"] is not None:
            np.testing.assert_array_equal(n_acc, case.ri["planted_len"])
    fwds = {}
    for b in range(cfg.nb):
        for c in range(cfg.nc):
            ref = case.oracle_verify(b, c, heads)
            fwds[b, c] = ref
            tag = f"{cfg.name}[b{b},c{c}]"
            assert_f32_close(f[b, c], ref["f"], tag + " f")
            assert_f32_close(s[b, c], ref["s"], tag + " s")
            assert_out_close(cfg, y[b, c], ref["y"], tag + " y")
            oo = o[b, c] if heads is None else o[b, c][:, heads]
            assert_out_close(cfg, oo, ref["o"], tag + " o")

    say(f"{cfg.name} slice")
    case.run_slice()
    torch.cuda.synchronize()
    snap = case.st.snapshot()
    for b in range(cfg.nb):
        cs = int(r_best[b])
        k = int(r_acc[b, cs])
        st = case.oracle_state(b)
        bn = case.blk_np
        new = oracle.slice_state(st, bn["x"][b, cs], fwds[b, cs], bn["k"][b, cs], bn["v"][b, cs], k)
        tag = f"{cfg.name}[b{b}] slice k={k} c*={cs}"
        assert int(snap["kv_len"][b]) == cfg.kv_lens[b] + k + 1, tag
        np.testing.assert_array_equal(f64(snap["short_win"][b]), new.short_win, err_msg=tag)
        assert_f32_close(snap["outer_win"][b], new.outer_win, tag + " outer_win")
        assert_f32_close(snap["iir"][b], new.iir, tag + " iir")
        kr, vr = case.st.read_rows(b, cfg.kv_lens[b], k + 1)
        np.testing.assert_array_equal(dv.to_host(kr), np.asarray(bn["k"][b, cs][: k + 1]).transpose(1, 0, 2))
        np.testing.assert_array_equal(dv.to_host(vr), np.asarray(bn["v"][b, cs][: k + 1]).transpose(1, 0, 2))
        if cfg.kv_lens[b] > 0:        # committed rows before the new ones are untouched
            kr0, _ = case.st.read_rows(b, cfg.kv_lens[b] - 1, 1)
            np.testing.assert_array_equal(dv.to_host(kr0)[:, 0], case.prefix_host[b][0][:, -1])
    return n_acc


def test_tiny_tiny_fp32_sampling():
    _check_round(Case(synth.CONFIGS["tiny"]))


def test_tiny_tiny_fp32_greedy():
    _check_round(Case(synth.scaled(synth.CONFIGS["tiny"], mode="greedy")))


@pytest.mark.parametrize("k", [0, 3, 6])
def test_tiny_forced_k_fig1(k):
    """Figure 1(c)/(d) shape: gamma = 6 with a planted accepted length."""
    _check_round(Case(synth.scaled(synth.CONFIGS["tiny"], mode="greedy"), forced_len=[k]))


def test_tiny_needles():
    _check_round(Case(synth.CONFIGS["tiny"], needle="self"))
    _check_round(Case(synth.CONFIGS["tiny"], needle="future"))


def test_mid8k_mid_bf16_sampling():
    _check_round(Case(synth.CONFIGS["mid8k"]))


@pytest.mark.parametrize("needle", ["self", "future"])
def test_mid8k_needles(needle):
    _check_round(Case(synth.CONFIGS["mid8k"], needle=needle))


@pytest.mark.parametrize("L", [0, 1, 31, 33, 1000])
def test_ragged_and_empty_prefix(L):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(L,), heads=4, d=256)
    _check_round(Case(cfg, needle="self"))


def test_gamma_zero_and_max_block():
    _check_round(Case(synth.scaled(synth.CONFIGS["mid8k"], gamma=0, kv_lens=(500,), heads=2, d=128)))
    _check_round(Case(synth.scaled(synth.CONFIGS["mid8k"], gamma=63, kv_lens=(777,), heads=2, d=128)))


def test_head_dim_64_bf16():
    _check_round(Case(synth.scaled(synth.CONFIGS["mid8k"], head_dim=64, heads=4, d=256, kv_lens=(3000,)), needle="self"))


def test_capacity_edge_exactly_full():
    cfg = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(1011,), heads=2, d=128)   # 1011 + 13 = 1024 = kv_cap
    _check_round(Case(cfg, kv_cap=1024))


@pytest.mark.parametrize("name", ["long262k", "long262k_g6"])
def test_long262k_long_context_full_size(name):
    _check_round(Case(synth.CONFIGS[name]))


def test_long262k_needles_full_size():
    _check_round(Case(synth.CONFIGS["long262k"], needle="self"))


def test_multi4x4_multi_candidate_ragged_full_size():
    _check_round(Case(synth.CONFIGS["multi4x4"]))


def test_multi4x4_recursive_acceptance_full_size():
    """The 4-candidate workload with lossless recursive acceptance over the candidates."""
    _check_round(Case(synth.scaled(synth.CONFIGS["multi4x4"], mode="recursive")))


def test_recursive_acceptance_shared_prefixes_round():
    """Small vocabulary: candidates share drafted prefixes, so the kept path can belong to any of them."""
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], mode="recursive", vocab=4, kv_lens=(333, 31, 1024, 0), cfg_id=41)
    _check_round(Case(cfg))


def test_multi4x4_needles():
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], kv_lens=(100, 2047, 5000, 64))
    _check_round(Case(cfg, needle="self"))


@pytest.mark.parametrize("nc,gamma", [(2, 15), (3, 10)])
def test_query_count_at_the_ring_boundary(nc, gamma):
    """32 queries per sequence (two 16-query tiles in registers) and 33 (the LDS-ring stream with
    its larger work items); needles make the prefix and block parts visible."""
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], nc=nc, gamma=gamma, kv_lens=(5000, 1234), heads=2, d=128)
    assert nc * (gamma + 1) in (32, 33)
    _check_round(Case(cfg, needle="self"))


def test_many_sequences_ragged():
    """Twelve sequences with ragged and empty prefixes: the work-list table holds every
    sequence's per-phase items, and the finish kernel locates them all."""
    lens = (0, 1, 31, 32, 33, 700, 2048, 4099, 9000, 12345, 64, 5)
    cfg = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=lens, heads=2, d=128, cfg_id=77)
    _check_round(Case(cfg, needle="self"))


def test_verify_is_deterministic_and_leaves_state_untouched():
    case = Case(synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(4321,)))
    say("determinism: verify twice")
    before = case.st.snapshot()
    case.run_verify()
    torch.cuda.synchronize()
    first = [dv.to_host(t).copy() for t in (case.blk.f, case.blk.s, case.blk.y, case.blk.o)]
    case.run_verify()
    torch.cuda.synchronize()
    second = [dv.to_host(t) for t in (case.blk.f, case.blk.s, case.blk.y, case.blk.o)]
    for a, b in zip(first, second):
        np.testing.assert_array_equal(a, b)
    after = case.st.snapshot()
    for key in before:
        np.testing.assert_array_equal(before[key], after[key])


def test_kv_write_read_roundtrip():
    cfg = synth.scaled(synth.CONFIGS["mid8k"], heads=3, kv_lens=(0,))
    lay = dv.DeviceLayer(cfg, synth.make_layer(cfg))
    st = dv.DeviceState(lay, 2, 256)
    say("kv write/read round trip")
    rows = torch.randn((3, 77, 128), device="cuda").to(torch.bfloat16)
    vals = torch.randn((3, 77, 128), device="cuda").to(torch.bfloat16)
    st.write_prefix(1, rows, vals, row0=45)
    k, v = st.read_rows(1, 45, 77)
    torch.cuda.synchronize()
    assert torch.equal(k, rows) and torch.equal(v, vals)
