"""GPU prefill (prompt -> committed state) against the fp64 oracle.

The oracle's prefill is pinned to the prompt's sequential single-position
steps (tests/test_oracle_prefill.py).  Sizes span one and several 256-position
chunks with ragged ends; the long prompt runs at the 262144-token size with
the oracle on a channel sample; the chained case checks that verify consumes
the state prefill writes.  Tolerances as in gpu_harness.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import assert_f32_close, assert_out_close, f64, say

pytestmark = pytest.mark.gpu


def _layer_state(cfg, L0, kv_cap, seed=0):
    params = synth.make_layer(cfg, seed)
    small = synth.make_state_small(cfg, seed)
    lay = dv.DeviceLayer(cfg, params)
    st = dv.DeviceState(lay, cfg.nb, kv_cap)
    st.load_small(small)
    pre = []
    for b in range(cfg.nb):
        kp = synth.kv_prefix(cfg, b, "k", seed, device="cuda", length=L0)
        vp = synth.kv_prefix(cfg, b, "v", seed, device="cuda", length=L0)
        if L0:
            st.write_prefix(b, kp, vp)
        pre.append((dv.to_host(kp), dv.to_host(vp)))
    st.kv_len.fill_(L0)
    return params, small, lay, st, pre


def _run_prefill(lay, st, cfg, T, L0, pr, want_y=True):
    at = hci.act_torch_dtype(lay.act)
    y = torch.empty((cfg.nb, T, cfg.d), dtype=at, device="cuda") if want_y else None
    ws = torch.empty(max(hci.prefill_workspace_bytes(lay.c, cfg.nb, T, want_y), 256), dtype=torch.uint8, device="cuda")
    hci.prefill(lay.c, st.c, cfg.nb, T, L0, pr["x"], pr["k"], pr["v"], y, ws)
    return y


def _check(cfg, T, L0, chans=None, seed=0, want_y=True):
    kv_cap = (L0 + T + 31) // 32 * 32 + 32
    params, small, lay, st, pre = _layer_state(cfg, L0, kv_cap, seed)
    pr = synth.prompt(cfg, T, seed, device="cuda")
    say(f"prefill {cfg.name} d={cfg.d} To={cfg.taps_outer} T={T} L0={L0} want_y={want_y}")
    y = _run_prefill(lay, st, cfg, T, L0, pr, want_y)
    torch.cuda.synchronize()
    snap = st.snapshot()
    yh = dv.to_host(y) if want_y else None
    chs = slice(None) if chans is None else chans
    for b in range(cfg.nb):
        sub = lambda a: np.asarray(a)[..., chs] if chans is not None else np.asarray(a)
        lay_o = oracle.Layer(params["w_short"][:, chs], params["w_outer"][:, chs], params["lam"][chs],
                             params["beta"][chs], params["c"][chs])
        st_o = oracle.SeqState(small["short_win"][b][:, chs], small["outer_win"][b][:, chs], small["iir"][b][chs],
                               [np.zeros((1, L0, 1))], [np.zeros((1, L0, 1))])
        xb = dv.to_host(pr["x"][b])[:, chs]
        new, yo = oracle.prefill_state(lay_o, st_o, xb, np.zeros((T, 1, 1)), np.zeros((T, 1, 1)), long=T > 2048)
        tag = f"prefill {cfg.name} T={T} b={b}"
        np.testing.assert_array_equal(f64(snap["short_win"][b][:, chs]), new.short_win, err_msg=tag)
        assert_f32_close(snap["outer_win"][b][:, chs], new.outer_win, tag + " outer_win")
        assert_f32_close(snap["iir"][b][chs], new.iir, tag + " iir")
        if want_y:
            assert_out_close(cfg, yh[b][:, chs], yo, tag + " y")
        assert int(snap["kv_len"][b]) == L0 + T
        kr, vr = st.read_rows(b, L0, T)
        assert torch.equal(kr, pr["k"][b].transpose(0, 1).contiguous()), tag + " k rows"
        assert torch.equal(vr, pr["v"][b].transpose(0, 1).contiguous()), tag + " v rows"
        if L0:
            k0, _ = st.read_rows(b, 0, L0)
            np.testing.assert_array_equal(dv.to_host(k0), pre[b][0])


# want_y=False with T >= To takes the folded state-only path; the others the chunked output path
@pytest.mark.parametrize("want_y", [True, False])
@pytest.mark.parametrize("T", [1, 5, 7, 8, 255, 256, 257, 1000])
def test_prefill_fp32_tiny_layer(T, want_y):
    _check(synth.CONFIGS["tiny"], T, L0=100, want_y=want_y)


@pytest.mark.parametrize("want_y", [True, False])
@pytest.mark.parametrize("T", [1, 13, 128, 129, 300, 4096, 9000])
def test_prefill_bf16_layer(T, want_y):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=512, heads=4, kv_lens=(0, 0))
    _check(cfg, T, L0=37, want_y=want_y)


@pytest.mark.parametrize("want_y", [True, False])
def test_prefill_short_taps_and_few_poles(want_y):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=48, heads=1, taps_short=1, taps_outer=2, poles=5, kv_lens=(0,))
    _check(cfg, 700, L0=0, want_y=want_y)


@pytest.mark.parametrize("want_y", [True, False])
def test_prefill_odd_channel_groups(want_y):
    """d not a multiple of the 64-channel scan group, 4 short taps, outer taps = 1."""
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=96, heads=1, taps_short=4, taps_outer=1, poles=16, kv_lens=(0,))
    _check(cfg, 3001, L0=5, want_y=want_y)


# The matrix-core outputs pass covers outer filters of up to 145 taps in 1..5 window steps of 32
# inputs (the window is To - 1 rounded up to 8, plus 16): each step count once, ragged prompt
# lengths, short filters of 2..4 taps, few and many poles, two sequences, a last channel group
# of 8 channels (d = 40); 160 taps take the chunked output path.
@pytest.mark.parametrize("To,Ts,N,T,d", [
    (7, 2, 3, 700, 40),        # one step
    (17, 4, 16, 513, 40),      # one step, the window exactly 32 inputs
    (40, 3, 16, 1000, 48),     # two steps
    (81, 4, 5, 257, 40),       # three steps
    (100, 2, 16, 999, 40),     # four steps
    (145, 3, 16, 2000, 48),    # five steps, the longest filter of the pass
    (160, 3, 16, 700, 40),     # past the pass: the chunked output path
])
def test_prefill_outputs_every_window_length(To, Ts, N, T, d):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=d, heads=1, taps_short=Ts, taps_outer=To, poles=N, kv_lens=(0, 0))
    _check(cfg, T, L0=11, want_y=True)


@pytest.mark.parametrize("want_y", [True, False])
def test_prefill_long_prompt_262k_channel_sample(want_y):
    """A channel sample that covers every XCD at both ends of the channel range: workgroups go to
    the eight XCDs round robin, channel group fastest (16-channel groups on the output path, 64 on
    the state path), so the first and last eight groups of either size land on every XCD."""
    cfg = synth.scaled(synth.CONFIGS["long262k"], kv_lens=(0,))
    ends = [16 * k for k in range(8)] + [64 * k + 63 for k in range(8)]
    chans = np.unique(np.array([0, 1, 63, 64, 777, 2048] + ends + [cfg.d - 1 - c for c in ends]))
    _check(cfg, 262144, L0=0, chans=chans, want_y=want_y)


@pytest.mark.parametrize("want_y", [True, False])
def test_prefill_chunks_compose_on_gpu(want_y):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=256, heads=2, kv_lens=(0,))
    T1, T2 = 1000, 3000
    kv_cap = 4096
    _, _, lay, st_a, _ = _layer_state(cfg, 0, kv_cap)
    _, _, _, st_b, _ = _layer_state(cfg, 0, kv_cap)
    pr = synth.prompt(cfg, T1 + T2, 3, device="cuda")
    say(f"prefill composition want_y={want_y}")
    y_full = _run_prefill(lay, st_a, cfg, T1 + T2, 0, pr, want_y)
    p1 = {n: t[:, :T1].contiguous() for n, t in pr.items()}
    p2 = {n: t[:, T1:].contiguous() for n, t in pr.items()}
    y1 = _run_prefill(lay, st_b, cfg, T1, 0, p1, want_y)
    y2 = _run_prefill(lay, st_b, cfg, T2, T1, p2, want_y)
    torch.cuda.synchronize()
    a, b = st_a.snapshot(), st_b.snapshot()
    np.testing.assert_array_equal(a["short_win"], b["short_win"])
    assert_f32_close(a["outer_win"], b["outer_win"], "outer_win")
    assert_f32_close(a["iir"], b["iir"], "iir")
    np.testing.assert_array_equal(a["kv_len"], b["kv_len"])
    ka, va = st_a.read_rows(0, 0, T1 + T2)      # rows past kv_len are never written: compare the used ones
    kb, vb = st_b.read_rows(0, 0, T1 + T2)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    if want_y:
        assert_out_close(cfg, dv.to_host(torch.cat([y1, y2], dim=1)), f64(dv.to_host(y_full)), "y")


def test_prefill_then_verify_round():
    """verify, accept and slice run from the state prefill leaves, against the oracle from its prefill."""
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=512, heads=4, kv_lens=(0,), mode="greedy")
    T = 2000
    params, small, lay, st, _ = _layer_state(cfg, 0, 2048 + 64)
    pr = synth.prompt(cfg, T, 5, device="cuda")
    say("prefill then verify")
    _run_prefill(lay, st, cfg, T, 0, pr, want_y=False)
    tables = synth.make_tables(cfg)
    anchor = synth.anchors(cfg)
    ri = synth.round_inputs(cfg, anchor)
    bn = synth.gather_block(cfg, tables, ri["tokens"])
    blk = dv.DeviceBlock(lay, 1, 1, cfg.gamma)
    blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
    dv.verify(lay, st, blk, T)
    torch.cuda.synchronize()
    st_o = oracle.SeqState(small["short_win"][0], small["outer_win"][0], small["iir"][0],
                           [np.zeros((cfg.heads, 0, cfg.head_dim))], [np.zeros((cfg.heads, 0, cfg.head_dim))])
    lay_o = oracle.Layer.from_dict(params)
    new, _ = oracle.prefill_state(lay_o, st_o, dv.to_host(pr["x"][0]), dv.to_host(pr["k"][0]), dv.to_host(pr["v"][0]))
    ref = oracle.verify_block(lay_o, new, bn["x"][0, 0], bn["q"][0, 0], bn["k"][0, 0], bn["v"][0, 0])
    assert_f32_close(dv.to_host(blk.s)[0, 0], ref["s"], "s after prefill")
    assert_out_close(cfg, dv.to_host(blk.y)[0, 0], ref["y"], "y after prefill")
    assert_out_close(cfg, dv.to_host(blk.o)[0, 0], ref["o"], "o after prefill")


def test_full_width_prefill_then_verify_round():
    """The 8192-token workload's layer (d = 4096, 32 x 128 heads) started from the state a prefill
    of an 8192-token prompt leaves instead of a drawn one: verify against the oracle's prefill."""
    cfg = synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(0,), mode="greedy")
    T = 8192
    params, small, lay, st, _ = _layer_state(cfg, 0, T + 64)
    pr = synth.prompt(cfg, T, 6, device="cuda")
    say("full-width prefill then verify")
    _run_prefill(lay, st, cfg, T, 0, pr, want_y=False)
    tables = synth.make_tables(cfg)
    ri = synth.round_inputs(cfg, synth.anchors(cfg))
    bn = synth.gather_block(cfg, tables, ri["tokens"])
    blk = dv.DeviceBlock(lay, 1, 1, cfg.gamma)
    blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
    dv.verify(lay, st, blk, T)
    torch.cuda.synchronize()
    st_o = oracle.SeqState(small["short_win"][0], small["outer_win"][0], small["iir"][0],
                           [np.zeros((cfg.heads, 0, cfg.head_dim))], [np.zeros((cfg.heads, 0, cfg.head_dim))])
    lay_o = oracle.Layer.from_dict(params)
    new, _ = oracle.prefill_state(lay_o, st_o, dv.to_host(pr["x"][0]), dv.to_host(pr["k"][0]), dv.to_host(pr["v"][0]),
                                  long=True)
    ref = oracle.verify_block(lay_o, new, bn["x"][0, 0], bn["q"][0, 0], bn["k"][0, 0], bn["v"][0, 0])
    assert_f32_close(dv.to_host(blk.f)[0, 0], ref["f"], "f after prefill")
    assert_f32_close(dv.to_host(blk.s)[0, 0], ref["s"], "s after prefill")
    assert_out_close(cfg, dv.to_host(blk.y)[0, 0], ref["y"], "y after prefill")
    assert_out_close(cfg, dv.to_host(blk.o)[0, 0], ref["o"], "o after prefill")
