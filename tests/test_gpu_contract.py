"""GPU block-forward / state-restoration contract and the sustained decode loop.

EvSpark digest (Interpretation; Figure 1(d)): one block forward plus a slice
at k restores the same state as k+1 sequential single-position steps, with
no replay.  On the GPU: windows, IIR state, KV rows and lengths bit for bit,
f / s / y of positions <= k bit for bit (identical per-position arithmetic),
attention outputs within the bf16 / fp32 output tolerance (the split-K
partition of the prefix differs between the two).

The sustained loop runs the wide layer (d = 8192, 64 heads, 131072-token
prefix) for 256 verify -> accept -> slice rounds with greedy drafts that
agree with the target for a Geometric(0.7) prefix, and checks state equality
against GPU sequential decoding every round, the conv/IIR state against the
fp64 oracle every round, and attention outputs against the oracle on a
sample of rounds and heads.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import Case, assert_f32_close, assert_out_close, f64, say

pytestmark = pytest.mark.gpu


def _clone_state(src: dv.DeviceState) -> dv.DeviceState:
    st = dv.DeviceState(src.layer, src.nb, src.kv_cap)
    for a in ("short_win", "outer_win", "iir", "k_cache", "v_cache", "kv_len"):
        getattr(st, a).copy_(getattr(src, a))
    return st


def _sequential(case: Case, st: dv.DeviceState, blk1: dv.DeviceBlock, acc1: dv.DeviceAccept, b: int, c: int,
                count: int, base_len: int):
    """count single-position steps (verify gamma=0 + slice at 0) over block rows 0..count-1."""
    outs = {"f": [], "s": [], "y": [], "o": []}
    for i in range(count):
        for name in ("x", "q", "k", "v"):
            src = getattr(case.blk, name)
            getattr(blk1, name).zero_()
            getattr(blk1, name)[b, 0, 0].copy_(src[b, c, i])
        dv.verify(case.lay, st, blk1, base_len + i)
        acc1.n_acc.zero_()
        dv.slice_state(case.lay, st, blk1, acc1, base_len + i)
        for name in outs:
            outs[name].append(dv.to_host(getattr(blk1, name))[b, 0, 0])
    return {k: np.stack(v) for k, v in outs.items()}


@pytest.mark.parametrize("cfgname,L", [("tiny", 256), ("mid8k", 1000), ("mid8k", 8192)])
def test_block_plus_slice_equals_sequential_steps(cfgname, L):
    cfg = synth.scaled(synth.CONFIGS[cfgname], kv_lens=(L,), mode="greedy")
    base = Case(cfg, host_prefix=False)
    say(f"contract {cfgname} L={L}: block verify")
    base.run_verify()
    torch.cuda.synchronize()
    f, s, y, o = (dv.to_host(t)[0, 0] for t in (base.blk.f, base.blk.s, base.blk.y, base.blk.o))
    blk1 = dv.DeviceBlock(base.lay, 1, 1, 0)
    acc1 = dv.DeviceAccept(1, 1, 0, cfg.vocab)
    for k in range(cfg.gamma + 1):
        say(f"contract {cfgname} L={L}: k={k}")
        blk_state = _clone_state(base.st)
        base.acc.n_acc.fill_(k)
        dv.slice_state(base.lay, blk_state, base.blk, base.acc, L)
        seq_state = _clone_state(base.st)
        outs = _sequential(base, seq_state, blk1, acc1, 0, 0, k + 1, L)
        torch.cuda.synchronize()
        a, bsnap = blk_state.snapshot(), seq_state.snapshot()
        for key in a:
            np.testing.assert_array_equal(a[key], bsnap[key], err_msg=f"k={k} {key}")
        for cache in ("k_cache", "v_cache"):    # bitwise: rows past kv_len hold whatever the allocator left
            assert torch.equal(getattr(blk_state, cache).view(torch.uint8),
                               getattr(seq_state, cache).view(torch.uint8)), f"k={k} {cache}"
        np.testing.assert_array_equal(f[: k + 1], outs["f"])
        np.testing.assert_array_equal(s[: k + 1], outs["s"])
        np.testing.assert_array_equal(y[: k + 1], outs["y"])
        assert_out_close(cfg, o[: k + 1], f64(outs["o"]), f"k={k} o")
        del blk_state, seq_state


def test_abandoned_round_can_be_verified_again():
    """Verify never commits: verify, skip slice, verify again -> identical outputs."""
    case = Case(synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(3000,)), host_prefix=False)
    say("abandoned round")
    case.run_verify()
    torch.cuda.synchronize()
    o1 = dv.to_host(case.blk.o).copy()
    case.run_verify()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o1, dv.to_host(case.blk.o))


SUSTAINED_ROUNDS = int(os.environ.get("HCI_SUSTAINED_ROUNDS", "256"))
ATTN_ROUNDS = {0, 1, 63, 127, 255}
# the first and last eight heads (the first and last items of every phase of the prefix work list,
# and every residue of the workgroup -> XCD round robin at both ends) and two in between
ATTN_HEADS = list(range(8)) + [17, 42] + list(range(56, 64))


def test_wide131k_sustained_loop_state_equality():
    cfg = synth.CONFIGS["wide131k"]
    say(f"wide131k set-up: d={cfg.d} H={cfg.heads} L={cfg.kv_lens[0]}")
    case = Case(cfg, host_prefix=False)
    kp = synth.kv_prefix(cfg, 0, "k", 0, device="cuda")
    vp = synth.kv_prefix(cfg, 0, "v", 0, device="cuda")
    pre_k = dv.to_host(kp[ATTN_HEADS])
    pre_v = dv.to_host(vp[ATTN_HEADS])
    del kp, vp
    seq = _clone_state(case.st)
    blk1 = dv.DeviceBlock(case.lay, 1, 1, 0)
    acc1 = dv.DeviceAccept(1, 1, 0, cfg.vocab)
    layer = oracle.Layer.from_dict(case.params)
    ost = oracle.SeqState(case.small["short_win"][0], case.small["outer_win"][0], case.small["iir"][0],
                          [pre_k], [pre_v])
    anchor = case.anchor.copy()
    L = cfg.kv_lens[0]
    ks = []
    for r in range(SUSTAINED_ROUNDS):
        ri = synth.round_inputs(cfg, anchor, r)
        bn = synth.gather_block(cfg, case.tables, ri["tokens"])
        case.blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
        case.acc.set_inputs(ri["target_logits"], ri["drafts"])
        if r % 32 == 0:
            say(f"wide131k round {r} L={L}")
        dv.verify(case.lay, case.st, case.blk, L)
        dv.accept(case.acc, hci.GREEDY)
        dv.slice_state(case.lay, case.st, case.blk, case.acc, L)
        torch.cuda.synchronize()
        k = int(dv.to_host(case.acc.n_acc)[0, 0])
        nxt = int(dv.to_host(case.acc.next)[0, 0])
        rk, rn, _ = oracle.greedy_accept(ri["target_logits"][0, 0], ri["drafts"][0, 0])
        assert (k, nxt) == (rk, rn), f"round {r}"
        ks.append(k)
        # sequential decoding of the same k+1 tokens on the GPU
        outs = _sequential(case, seq, blk1, acc1, 0, 0, k + 1, L)
        torch.cuda.synchronize()
        a, b = case.st.snapshot(), seq.snapshot()
        for key in a:
            np.testing.assert_array_equal(a[key], b[key], err_msg=f"round {r} {key}")
        kr_a, vr_a = case.st.read_rows(0, L, k + 1)
        kr_b, vr_b = seq.read_rows(0, L, k + 1)
        assert torch.equal(kr_a, kr_b) and torch.equal(vr_a, vr_b), f"round {r} kv rows"
        np.testing.assert_array_equal(dv.to_host(case.blk.y)[0, 0, : k + 1], outs["y"])
        # oracle: conv/IIR state every round, attention on sampled rounds and heads
        x, q, kk, vv = bn["x"][0, 0], bn["q"][0, 0], bn["k"][0, 0], bn["v"][0, 0]
        fo = oracle.depthwise_fir(x, ost.short_win, layer.w_short)
        go = oracle.depthwise_fir(fo, ost.outer_win, layer.w_outer)
        so, yo = oracle.modal_iir(go, ost.iir, layer.lam, layer.beta, layer.c)
        assert_out_close(cfg, dv.to_host(case.blk.y)[0, 0], yo, f"round {r} y")
        if r in ATTN_ROUNDS:
            say(f"wide131k round {r}: oracle attention on heads {ATTN_HEADS}")
            oo = oracle.block_attention(q[:, ATTN_HEADS], kk[:, ATTN_HEADS], vv[:, ATTN_HEADS],
                                        ost.k_blocks, ost.v_blocks)
            assert_out_close(cfg, dv.to_host(case.blk.o)[0, 0][:, ATTN_HEADS], oo, f"round {r} o")
        ost = oracle.slice_state(ost, x, {"f": fo, "s": so}, kk[:, ATTN_HEADS], vv[:, ATTN_HEADS], k)
        snap = a
        np.testing.assert_array_equal(f64(snap["short_win"][0]), ost.short_win, err_msg=f"round {r}")
        assert_f32_close(snap["outer_win"][0], ost.outer_win, f"round {r} outer_win")
        assert_f32_close(snap["iir"][0], ost.iir, f"round {r} iir")
        L += k + 1
        assert int(snap["kv_len"][0]) == L
        anchor = np.array([nxt], np.int32)
    say(f"wide131k done: {len(ks)} rounds, mean k {np.mean(ks):.2f}, hist {np.bincount(ks, minlength=cfg.P)}")
    assert len(set(ks)) >= 5
