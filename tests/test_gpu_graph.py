"""A whole round -- hci_verify_block, hci_accept, hci_slice_state -- captured in
a HIP graph replays to the eager round's bits.  The verify's set-up kernel
clears the job queue's counter (no memset is recorded), and the workspace is
allocated before the capture.  Between replays the committed state and every
output are restored or cleared by eager work, and each replay is compared with
the eager round: outputs y, o, f, s, the accepted counts, next tokens and best
candidate, and the new committed state (windows, IIR state, KV caches,
lengths)."""
from __future__ import annotations

import pytest
import torch

from gpu_harness import Case, say
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth

pytestmark = pytest.mark.gpu

STATE = ("short_win", "outer_win", "iir", "k_cache", "v_cache", "kv_len")


def _round(case, mode, bound, stream):
    dv.verify(case.lay, case.st, case.blk, bound, stream=stream)
    dv.accept(case.acc, mode, case.cfg.temperature, stream=stream)
    dv.slice_state(case.lay, case.st, case.blk, case.acc, bound, stream=stream)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),                                                          # fp32 layer, per-item prefix kernel
    ("mid8k", dict(kv_lens=(3000,), heads=4, d=256)),                      # one query tile, sampling
    ("multi4x4", dict(kv_lens=(333, 1000, 64, 2047), heads=2, d=128)),     # four query tiles, best candidate
])
def test_round_graph_replay_equals_eager(name, kw):
    cfg = synth.scaled(synth.CONFIGS[name], **kw)
    case = Case(cfg, host_prefix=False)
    mode = hci.GREEDY if cfg.mode == "greedy" else hci.SAMPLE
    bound = cfg.max_kv_len
    saved = {n: getattr(case.st, n).clone() for n in STATE}
    outs = {"y": case.blk.y, "o": case.blk.o, "f": case.blk.f, "s": case.blk.s,
            "n_acc": case.acc.n_acc, "next": case.acc.next, "best": case.acc.best}
    outs.update({n: getattr(case.st, n) for n in STATE})

    def restore():
        for n in STATE:
            getattr(case.st, n).copy_(saved[n])
        for n in ("y", "o", "f", "s", "n_acc", "next", "best"):
            outs[n].zero_()

    say(f"graph {name}: eager round")
    _round(case, mode, bound, None)
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in outs.items()}
    assert int(eager["kv_len"].sum()) > sum(cfg.kv_lens)              # the round committed something

    say(f"graph {name}: capture")
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            _round(case, mode, bound, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        restore()
        torch.cuda.synchronize()
        say(f"graph {name}: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t.view(torch.uint8), eager[n].view(torch.uint8)), f"replay {rep}: {n}"
