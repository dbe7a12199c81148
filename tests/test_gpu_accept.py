"""GPU acceptance against the oracle over vocabulary sizes, temperatures, block
lengths and candidate counts the workloads do not cover (bit-exact k, next
token and best candidate; margins asserted away from rounding ties)."""
import numpy as np
import pytest
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _inputs(V, gamma, nb, nc, T, mode, seed):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], vocab=V, gamma=gamma, kv_lens=(0,) * nb, nc=nc, mode=mode,
                       temperature=T, cfg_id=100 + seed)
    anchor = synth.anchors(cfg, 0, seed)
    return cfg, synth.round_inputs(cfg, anchor, 0, seed)


_MODES = {"greedy": hci.GREEDY, "sample": hci.SAMPLE, "recursive": hci.SAMPLE_RECURSIVE}


def _run(cfg, ri, mode=None):
    acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    acc.set_inputs(ri["target_logits"], ri["drafts"], ri["draft_logits"], ri["uniforms"])
    dv.accept(acc, _MODES[mode or cfg.mode], cfg.temperature)
    torch.cuda.synchronize()
    return tuple(dv.to_host(t) for t in (acc.n_acc, acc.next, acc.best, acc.margin))


@pytest.mark.parametrize("V", [1, 3, 300, 513, 4099])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_accept_vocab_sizes(V, mode):
    for gamma, nc, T, seed in ((0, 1, 1.0, 1), (1, 3, 0.5, 2), (12, 2, 2.0, 3), (5, 1, 1.0, 4)):
        cfg, ri = _inputs(V, gamma, 2, nc, T, mode, seed)
        say(f"accept V={V} {mode} gamma={gamma} nc={nc} T={T}")
        n_acc, nxt, best, marg = _run(cfg, ri)
        r_acc, r_next, r_best, r_marg = oracle.accept_candidates(mode, ri["target_logits"], ri["draft_logits"],
                                                                 ri["drafts"], ri["uniforms"], T)
        if mode == "sample":
            assert (r_marg > 1e-12).all()
        np.testing.assert_array_equal(n_acc, r_acc)
        np.testing.assert_array_equal(nxt, r_next)
        np.testing.assert_array_equal(best, r_best)


def test_accept_draft_ids_out_of_range_count_as_rejection():
    cfg, ri = _inputs(64, 6, 1, 1, 1.0, "sample", 7)
    # make every draft acceptable (draft distribution = target distribution) except an invalid id at m=3
    ri["draft_logits"][:] = ri["target_logits"][:, :, :cfg.gamma]
    drafts = ri["drafts"].copy()
    drafts[0, 0, 2] = cfg.vocab + 5
    ri["drafts"] = drafts
    say("accept invalid draft id")
    n_acc, nxt, _, _ = _run(cfg, ri)
    assert int(n_acc[0, 0]) == 2
    assert 0 <= int(nxt[0, 0]) < cfg.vocab
    drafts[0, 0, 2] = -1
    n_acc, _, _, _ = _run(cfg, ri)
    assert int(n_acc[0, 0]) == 2


def test_accept_full_acceptance_and_greedy_bonus():
    cfg, ri = _inputs(512, 12, 3, 2, 1.0, "sample", 8)
    ri["draft_logits"][:] = ri["target_logits"][:, :, :cfg.gamma]     # q == p: always accept
    say("accept q == p")
    n_acc, nxt, best, _ = _run(cfg, ri)
    assert (n_acc == cfg.gamma).all() and (best == 0).all()
    _, r_next, _, _ = oracle.accept_candidates("sample", ri["target_logits"], ri["draft_logits"], ri["drafts"],
                                              ri["uniforms"], 1.0)
    np.testing.assert_array_equal(nxt, r_next)


# ------------------------------------------------- recursive acceptance over several candidates

def _check_recursive(cfg, zt, zd, drafts, u):
    ri = {"target_logits": zt, "draft_logits": zd, "drafts": drafts, "uniforms": u}
    n_acc, nxt, best, marg = _run(cfg, ri, "recursive")
    r_acc, r_next, r_best, r_marg = oracle.accept_candidates("recursive", zt, zd, drafts, u, cfg.temperature)
    assert (r_marg > 1e-12).all()
    np.testing.assert_array_equal(best, r_best)
    np.testing.assert_array_equal(n_acc, r_acc)
    np.testing.assert_array_equal(nxt, r_next)
    return n_acc, best


@pytest.mark.parametrize("V,nc,gamma,T", [(3, 4, 12, 1.0), (8, 4, 6, 0.5), (300, 2, 12, 1.0), (513, 4, 1, 2.0),
                                          (4099, 3, 12, 1.0), (5, 64, 0, 1.0), (6, 5, 12, 0.7)])
def test_recursive_prefix_keyed_inputs(V, nc, gamma, T):
    """Rows keyed by the prefix: candidates that share drafts share rows, so alive sets grow past one."""
    nb = 3
    deep = 0
    for seed in range(3):
        cfg = synth.scaled(synth.CONFIGS["multi4x4"], vocab=V, gamma=gamma, kv_lens=(0,) * nb, nc=nc, mode="sample",
                           temperature=T, cfg_id=300 + seed)
        zt, zd, drafts, u = synth.prefix_keyed_round(cfg, 0, seed, scale=3.0 if V < 10 else 1.4)
        say(f"recursive prefix-keyed V={V} nc={nc} gamma={gamma} T={T} seed={seed}")
        n_acc, best = _check_recursive(cfg, zt, zd, drafts, u)
        deep += int((n_acc >= 1).sum(axis=1).max() > 1) if gamma else 0
    if V < 10 and nc > 1 and gamma > 1:
        assert deep > 0            # some sequence kept more than one candidate alive past depth 1


@pytest.mark.parametrize("nc", [1, 2, 4])
def test_recursive_independent_candidate_rows(nc):
    """Random rows per candidate (the caller's rows need not agree): the rule still takes the rep's rows."""
    for V, gamma, T, seed in ((64, 12, 1.0, 1), (512, 6, 0.5, 2), (2, 3, 1.0, 3)):
        cfg, ri = _inputs(V, gamma, 2, nc, T, "sample", seed)
        say(f"recursive independent rows V={V} nc={nc} gamma={gamma}")
        _check_recursive(cfg, ri["target_logits"], ri["draft_logits"], ri["drafts"], ri["uniforms"])


def test_recursive_one_candidate_is_sample_mode_bitwise():
    for V, gamma, T, seed in ((512, 12, 1.0, 4), (7, 1, 0.5, 5), (4099, 6, 2.0, 6), (33, 0, 1.0, 7)):
        cfg, ri = _inputs(V, gamma, 4, 1, T, "sample", seed)
        say(f"recursive nc=1 vs sample V={V} gamma={gamma}")
        a = _run(cfg, ri, "recursive")
        b = _run(cfg, ri, "sample")
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_recursive_invalid_ids_and_full_acceptance():
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], vocab=64, gamma=6, kv_lens=(0,), nc=3, mode="sample", cfg_id=320)
    zt, zd, drafts, u = synth.prefix_keyed_round(cfg, 0, 1)
    zd = zt[:, :, :cfg.gamma].copy()               # q == p everywhere: candidate 0 keeps every draft
    say("recursive q == p")
    n_acc, best = _check_recursive(cfg, zt, zd, drafts, u)
    assert int(best[0]) == 0 and int(n_acc[0, 0]) == cfg.gamma
    bad = drafts.copy()
    bad[0, 0, 0] = cfg.vocab + 3                  # candidate 0 invalid at depth 0: rejected, residual taken
    bad[0, 1, 0] = -1
    say("recursive invalid draft ids")
    _check_recursive(cfg, zt, zd, bad, u)
