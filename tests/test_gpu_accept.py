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
    cfg = synth.scaled(synth.CONFIGS["c2"], vocab=V, gamma=gamma, kv_lens=(0,) * nb, nc=nc, mode=mode,
                       temperature=T, cfg_id=100 + seed)
    anchor = synth.anchors(cfg, 0, seed)
    return cfg, synth.round_inputs(cfg, anchor, 0, seed)


def _run(cfg, ri):
    acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    acc.set_inputs(ri["target_logits"], ri["drafts"], ri["draft_logits"], ri["uniforms"])
    dv.accept(acc, hci.GREEDY if cfg.mode == "greedy" else hci.SAMPLE, cfg.temperature)
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
