"""The device status word and the guards behind it (include/hci.h, HCI_DS_*).

Values that only the device holds -- the logits acceptance reads, the k and c*
it hands to slicing, kv_len -- are checked by the kernels themselves: a value
out of contract sets a bit in the caller's per-sequence status word and never
commits state (nothing is clamped into range).  Every case here is one that the
kernels' own checks turn into a report, so every kernel runs to completion.
Also: a verify in which every prefix is empty reads no stale work list from a
reused or garbage-filled workspace.
"""
import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import Case, assert_out_close, f64, say

pytestmark = pytest.mark.gpu

TINY = synth.CONFIGS["tiny"]
_MODES = {"greedy": hci.GREEDY, "sample": hci.SAMPLE, "recursive": hci.SAMPLE_RECURSIVE}


def _state(case, rows=None):
    """Every part of the committed state of every sequence, copied to the host."""
    torch.cuda.synchronize()
    snap = case.st.snapshot()
    cfg = case.cfg
    out = {k: np.array(v, copy=True) for k, v in snap.items()}
    for b in range(cfg.nb):
        n = rows if rows is not None else cfg.kv_lens[b] + cfg.P
        kr, vr = case.st.read_rows(b, 0, n)
        out[f"k{b}"], out[f"v{b}"] = dv.to_host(kr), dv.to_host(vr)
    return out


def _same_state(a, b, tag):
    assert a.keys() == b.keys()
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{tag}: {k} changed")


def _status(case):
    torch.cuda.synchronize()
    return [int(v) & 0xFFFFFFFF for v in dv.to_host(case.st.status)]


def _accept(case, mode):
    dv.accept(case.acc, _MODES[mode], case.cfg.temperature, status=case.st.status)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("kind", ["nan", "posinf", "all_neginf"])
def test_nonfinite_target_row_commits_nothing(mode, kind):
    cfg = synth.scaled(TINY, mode=mode)
    case = Case(cfg)
    zt = case.ri["target_logits"].copy()
    if kind == "nan":
        zt[0, 0, 0, 17] = np.nan
    elif kind == "posinf":
        zt[0, 0, 0, 3] = np.inf
    else:
        zt[0, 0, 0, :] = -np.inf
    case.acc.set_inputs(zt, case.ri["drafts"], case.ri["draft_logits"], case.ri["uniforms"])
    before = _state(case)
    say(f"status: non-finite target row ({kind}, {mode})")
    case.run_verify()
    _accept(case, mode)
    case.run_slice()
    torch.cuda.synchronize()
    assert int(dv.to_host(case.acc.n_acc)[0, 0]) == -1
    assert int(dv.to_host(case.acc.next)[0, 0]) == -1
    assert int(dv.to_host(case.acc.best)[0]) == -1
    st = _status(case)[0]
    assert st == hci.DS_NONFINITE | hci.DS_K_RANGE, hci.device_status_string(st)
    _same_state(before, _state(case), f"non-finite {kind}")


def test_nonfinite_draft_row_in_sampling():
    case = Case(synth.scaled(TINY, mode="sample"))
    zd = case.ri["draft_logits"].copy()
    zd[0, 0, 0, 5] = np.nan                     # q_1, read by the first ratio test
    case.acc.set_inputs(case.ri["target_logits"], case.ri["drafts"], zd, case.ri["uniforms"])
    before = _state(case)
    say("status: NaN draft row")
    case.run_verify()
    _accept(case, "sample")
    case.run_slice()
    assert int(dv.to_host(case.acc.n_acc)[0, 0]) == -1
    assert _status(case)[0] == hci.DS_NONFINITE | hci.DS_K_RANGE
    _same_state(before, _state(case), "NaN draft row")


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_neginf_entries_are_valid_logits(mode):
    """-Inf is probability zero, not an error: the decision matches the oracle and nothing is reported."""
    cfg = synth.scaled(TINY, mode=mode)
    case = Case(cfg)
    zt = case.ri["target_logits"].copy()
    zd = None if case.ri["draft_logits"] is None else case.ri["draft_logits"].copy()
    rng = np.random.default_rng(5)
    for arr in [a for a in (zt, zd) if a is not None]:
        for r in range(arr.shape[2]):
            top = int(np.argmax(arr[0, 0, r]))
            cols = rng.choice(cfg.vocab, 40, replace=False)
            cols = cols[cols != top]
            arr[0, 0, r, cols] = -np.inf
            if mode == "sample":                # keep every draft token possible under q
                d = case.ri["drafts"][0, 0]
                if arr is zd and r < len(d):
                    arr[0, 0, r, d[r]] = case.ri["draft_logits"][0, 0, r, d[r]]
    case.acc.set_inputs(zt, case.ri["drafts"], zd, case.ri["uniforms"])
    say(f"status: -inf entries ({mode})")
    _accept(case, mode)
    torch.cuda.synchronize()
    r_acc, r_next, _, r_marg = oracle.accept_candidates(mode, zt, zd, case.ri["drafts"], case.ri["uniforms"],
                                                        cfg.temperature)
    assert (r_marg > 1e-12).all()
    np.testing.assert_array_equal(dv.to_host(case.acc.n_acc), r_acc)
    np.testing.assert_array_equal(dv.to_host(case.acc.next), r_next)
    assert _status(case) == [0]


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_draft_id_out_of_range_is_reported(mode):
    cfg = synth.scaled(TINY, mode=mode)
    case = Case(cfg, forced_len=None)
    drafts = case.ri["drafts"].copy()
    if mode == "greedy":
        drafts[0, 0, 0] = -7                      # the first comparison reads it
    else:
        # q = p makes every valid draft acceptable; the invalid id at m = 3 stops the block at k = 2
        case.ri["draft_logits"][:] = case.ri["target_logits"][:, :, : cfg.gamma]
        drafts[0, 0, 2] = cfg.vocab + 1
    case.acc.set_inputs(case.ri["target_logits"], drafts, case.ri["draft_logits"], case.ri["uniforms"])
    say(f"status: draft id out of range ({mode})")
    _accept(case, mode)
    torch.cuda.synchronize()
    k = int(dv.to_host(case.acc.n_acc)[0, 0])
    assert k == (0 if mode == "greedy" else 2)
    assert 0 <= int(dv.to_host(case.acc.next)[0, 0]) < cfg.vocab
    assert _status(case) == [hci.DS_DRAFT_ID]


@pytest.mark.parametrize("bad_k", [-2, "gamma+5"])
def test_slice_k_out_of_range_leaves_state(bad_k):
    case = Case(synth.scaled(TINY, mode="greedy"))
    case.run_verify()
    _accept(case, "greedy")
    torch.cuda.synchronize()
    assert _status(case) == [0]
    k = case.cfg.gamma + 5 if bad_k == "gamma+5" else bad_k
    case.acc.n_acc.fill_(k)
    before = _state(case)
    say(f"status: slice with k={k}")
    case.run_slice()
    assert _status(case) == [hci.DS_K_RANGE]
    _same_state(before, _state(case), f"k={k}")


@pytest.mark.parametrize("bad_c", [-1, 2])
def test_slice_candidate_out_of_range_leaves_state(bad_c):
    cfg = synth.scaled(TINY, nc=2, mode="greedy")
    case = Case(cfg)
    case.run_verify()
    _accept(case, "greedy")
    torch.cuda.synchronize()
    case.acc.best.fill_(bad_c)
    before = _state(case)
    say(f"status: slice with c*={bad_c}")
    case.run_slice()
    assert _status(case) == [hci.DS_CAND_RANGE]
    _same_state(before, _state(case), f"c*={bad_c}")


def test_bad_candidate_cannot_win_and_others_commit():
    """One of two candidates has a NaN logit: it is marked -1, the other wins and commits normally."""
    cfg = synth.scaled(TINY, nc=2, mode="greedy")
    case = Case(cfg)
    zt = case.ri["target_logits"].copy()
    zt[0, 1, 0, 0] = np.nan
    case.acc.set_inputs(zt, case.ri["drafts"], case.ri["draft_logits"], case.ri["uniforms"])
    say("status: NaN in one candidate of two")
    case.run_verify()
    _accept(case, "greedy")
    case.run_slice()
    torch.cuda.synchronize()
    n_acc = dv.to_host(case.acc.n_acc)
    r_acc, _, _, _ = oracle.accept_candidates("greedy", case.ri["target_logits"][:, :1], None,
                                              case.ri["drafts"][:, :1], None, 1.0)
    assert int(n_acc[0, 1]) == -1 and int(n_acc[0, 0]) == int(r_acc[0, 0])
    assert int(dv.to_host(case.acc.best)[0]) == 0
    assert _status(case) == [hci.DS_NONFINITE]
    assert int(dv.to_host(case.st.kv_len)[0]) == cfg.kv_lens[0] + int(r_acc[0, 0]) + 1


def test_recursive_nonfinite_marks_the_sequence():
    cfg = synth.scaled(TINY, nc=3, mode="recursive", vocab=8, cfg_id=71)
    case = Case(cfg)
    zt = case.ri["target_logits"].copy()
    zt[0, 0, 0, 1] = np.inf
    case.acc.set_inputs(zt, case.ri["drafts"], case.ri["draft_logits"], case.ri["uniforms"])
    before = _state(case)
    say("status: recursive acceptance with +Inf")
    case.run_verify()
    _accept(case, "recursive")
    case.run_slice()
    assert (dv.to_host(case.acc.n_acc) == -1).all() and (dv.to_host(case.acc.next) == -1).all()
    assert int(dv.to_host(case.acc.best)[0]) == -1
    assert _status(case) == [hci.DS_NONFINITE | hci.DS_CAND_RANGE]
    _same_state(before, _state(case), "recursive +Inf")


def test_kv_len_above_the_host_bound():
    """kv_len > max_kv_len: verify attends to the first max_kv_len keys and reports; slice commits nothing."""
    cfg = synth.scaled(TINY, mode="greedy")
    case = Case(cfg)
    lim = 200
    say("status: kv_len above max_kv_len")
    dv.verify(case.lay, case.st, case.blk, lim)
    torch.cuda.synchronize()
    assert _status(case) == [hci.DS_KV_LEN]
    kp, vp = case.prefix_host[0]
    st = oracle.SeqState(case.small["short_win"][0], case.small["outer_win"][0], case.small["iir"][0],
                         [kp[:, :lim]], [vp[:, :lim]])
    bn = case.blk_np
    ref = oracle.verify_block(oracle.Layer.from_dict(case.params), st, bn["x"][0, 0], bn["q"][0, 0],
                              bn["k"][0, 0], bn["v"][0, 0])
    assert_out_close(cfg, dv.to_host(case.blk.o)[0, 0], ref["o"], "o over the clamped prefix")
    _accept(case, "greedy")
    before = _state(case)
    dv.slice_state(case.lay, case.st, case.blk, case.acc, lim)
    assert _status(case) == [hci.DS_KV_LEN]
    _same_state(before, _state(case), "kv_len above bound")


def test_negative_kv_len_reads_as_empty():
    cfg = synth.scaled(TINY, mode="greedy")
    case = Case(cfg)
    case.st.kv_len.fill_(-3)
    say("status: negative kv_len")
    case.run_verify()
    torch.cuda.synchronize()
    assert _status(case) == [hci.DS_KV_LEN]
    st = oracle.SeqState(case.small["short_win"][0], case.small["outer_win"][0], case.small["iir"][0], [], [])
    bn = case.blk_np
    ref = oracle.verify_block(oracle.Layer.from_dict(case.params), st, bn["x"][0, 0], bn["q"][0, 0],
                              bn["k"][0, 0], bn["v"][0, 0])
    assert_out_close(cfg, dv.to_host(case.blk.o)[0, 0], ref["o"], "o with an empty prefix")


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("how", ["garbage", "reused"])
def test_empty_prefixes_ignore_workspace_contents(act, how):
    """max_kv_len = 0: the finish kernel reads the set-up kernel's empty work list, never the
    workspace's earlier contents (0xFF bytes, or a previous verify's list and partials)."""
    base = TINY if act == "f32" else synth.scaled(synth.CONFIGS["mid8k"], d=256, heads=2, kv_lens=(1000, 700))
    cfg = synth.scaled(base, mode="greedy")
    case = Case(cfg)
    ws = case.blk.ensure_workspace(cfg.max_kv_len)
    if how == "garbage":
        ws.fill_(0xFF)
    else:
        case.run_verify()                       # leaves a non-empty list and partials behind
    torch.cuda.synchronize()
    case.st.kv_len.zero_()
    say(f"status: empty prefixes after a {how} workspace ({act})")
    dv.verify(case.lay, case.st, case.blk, 0)
    torch.cuda.synchronize()
    o = dv.to_host(case.blk.o)
    bn = case.blk_np
    for b in range(cfg.nb):
        st = oracle.SeqState(case.small["short_win"][b], case.small["outer_win"][b], case.small["iir"][b], [], [])
        ref = oracle.verify_block(oracle.Layer.from_dict(case.params), st, bn["x"][b, 0], bn["q"][b, 0],
                                  bn["k"][b, 0], bn["v"][b, 0])
        assert_out_close(cfg, o[b, 0], ref["o"], f"o[b{b}] empty prefix")
    assert _status(case) == [0] * cfg.nb


@pytest.mark.parametrize("want_y", [False, True])
def test_prefill_skips_a_sequence_with_kv_len_out_of_contract(want_y):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=128, heads=2, kv_lens=(0, 0))
    T, lim = 300, 64
    params = synth.make_layer(cfg)
    small = synth.make_state_small(cfg)
    lay = dv.DeviceLayer(cfg, params)
    st = dv.DeviceState(lay, cfg.nb, (lim + T + 31) // 32 * 32 + 32)
    st.load_small(small)
    st.kv_len.copy_(torch.tensor([10, lim + 3], dtype=torch.int32))
    pr = synth.prompt(cfg, T, device="cuda")
    torch.cuda.synchronize()
    before = {k: np.array(v, copy=True) for k, v in st.snapshot().items()}
    k1_before, _ = st.read_rows(1, 0, lim + 3 + T)
    k1_before = dv.to_host(k1_before)
    at = hci.act_torch_dtype(lay.act)
    y = torch.empty((cfg.nb, T, cfg.d), dtype=at, device="cuda") if want_y else None
    ws = torch.empty(max(hci.prefill_workspace_bytes(lay.c, cfg.nb, T, want_y), 256), dtype=torch.uint8, device="cuda")
    say(f"status: prefill with one sequence out of contract (want_y={want_y})")
    hci.prefill(lay.c, st.c, cfg.nb, T, lim, pr["x"], pr["k"], pr["v"], y, ws)
    torch.cuda.synchronize()
    after = st.snapshot()
    assert [int(v) for v in dv.to_host(st.status)] == [0, hci.DS_KV_LEN]
    assert int(after["kv_len"][0]) == 10 + T and int(after["kv_len"][1]) == lim + 3
    for key in ("short_win", "outer_win", "iir"):
        np.testing.assert_array_equal(after[key][1], before[key][1], err_msg=key)
        assert not np.array_equal(after[key][0], before[key][0]), key
    k1_after, _ = st.read_rows(1, 0, lim + 3 + T)
    np.testing.assert_array_equal(dv.to_host(k1_after), k1_before)
    kr, _ = st.read_rows(0, 10, T)
    assert torch.equal(kr, pr["k"][0].transpose(0, 1).contiguous())
