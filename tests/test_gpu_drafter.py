"""GPU drafter against the fp64 oracle.

Serial sampling: bit-exact drafts and biased logits on the same fp32 logits
(margins asserted away from rounding ties).  Trunk: logits within the
layer-stack tolerance (2^-5 rms(ref) + 2^-6 |ref| elementwise; both sides
round the stored activations to bf16 from sums that differ in the last fp32
bits).  The whole draft (trunk + sampling) captured in a HIP graph replays
bit-identically to the eager calls.
"""
import numpy as np
import pytest
import torch

from oracle import drafter as OD
from hybrid_conv_iir_amd import drafter as ddr
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import say

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# every run length of the four-wave sampler (ids per thread 1, 2, 4, 8, 16), ragged last runs
@pytest.mark.parametrize("V,gamma,T", [(16, 1, 1.0), (512, 12, 1.0), (512, 32, 0.5), (4096, 6, 2.0), (33, 7, 1.0),
                                       (1000, 5, 1.0), (1537, 4, 0.75)])
def test_draft_sample_matches_oracle(V, gamma, T):
    nb = 3
    g = torch.Generator().manual_seed(V * 100 + gamma)
    z = torch.randn((nb, gamma, V), generator=g) * 2 ** 0.5
    B = torch.randn((V, V), generator=g)
    anchor = torch.randint(0, V, (nb,), generator=g, dtype=torch.int32)
    u = torch.rand((nb, gamma), generator=g, dtype=torch.float64)
    say(f"draft sample V={V} gamma={gamma} T={T}")
    dev = {n: t.cuda() for n, t in (("z", z), ("B", B), ("a", anchor), ("u", u))}
    drafts = torch.empty((nb, gamma), dtype=torch.int32, device="cuda")
    dl = torch.empty((nb, gamma, V), dtype=torch.float32, device="cuda")
    marg = torch.empty((nb, gamma), dtype=torch.float64, device="cuda")
    hci.draft_sample(nb, gamma, V, T, dev["z"], dev["B"], dev["a"], dev["u"], drafts, dl, marg)
    torch.cuda.synchronize()
    for b in range(nb):
        r_dr, r_dl, r_m = OD.draft_sample(z[b].numpy(), B.numpy(), int(anchor[b]), u[b].numpy(), T)
        assert (r_m > 1e-12).all()
        np.testing.assert_array_equal(drafts[b].cpu().numpy(), r_dr)
        np.testing.assert_array_equal(dl[b].cpu().numpy(), r_dl)


def _oracle_drafter(dc, p):
    L = [OD.TrunkLayer(g1=f64(x["g1"]), w_qkv=f64(x["w_qkv"]), w_o=f64(x["w_o"]), g2=f64(x["g2"]),
                       w_up=f64(x["w_up"]), w_down=f64(x["w_down"])) for x in p["layers"]]
    return OD.Drafter(w_proj=f64(p["w_proj"]), emb=f64(p["emb"]), mask=f64(p["mask"]),
                      markov=p["markov"].cpu().numpy(), layers=L, g_f=f64(p["g_f"]), heads=dc.heads, eps=dc.eps)


def _close(got, ref, tag):
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    ok = err <= 2.0 ** -5 * rms + 2.0 ** -6 * np.abs(ref)
    assert ok.all(), f"{tag}: {int((~ok).sum())} outside, max err / rms {err.max() / rms:.3g}"


@pytest.mark.parametrize("name,nb,gamma", [("d_small", 2, 12), ("d_small", 1, 1), ("d1k", 1, 12), ("d1k", 3, 6)])
def test_draft_logits_match_oracle(name, nb, gamma):
    dc = synth.DRAFTER_CONFIGS[name]
    p = synth.make_drafter(dc, 0, device="cuda")
    dd = ddr.DeviceDrafter(dc, p)
    rd = synth.draft_round(dc, nb, gamma, 0, 0, device="cuda")
    out = dd.buffers(nb, gamma)
    say(f"draft logits {name} nb={nb} gamma={gamma}")
    hci.draft_logits(dd.c, nb, gamma, rd["window"], rd["anchor"].cuda(), out["z"], dd.ws)
    torch.cuda.synchronize()
    od = _oracle_drafter(dc, p)
    for b in range(nb):
        ref = OD.draft_logits(od, f64(rd["window"][b]), int(rd["anchor"][b]), gamma)
        _close(f64(out["z"][b]), ref, f"{name}[b{b}] z")


def test_draft_graph_replay_equals_eager():
    dc = synth.DRAFTER_CONFIGS["d1k"]
    nb, gamma = 2, 12
    dd = ddr.DeviceDrafter(dc, synth.make_drafter(dc, 1, device="cuda"))
    rd = synth.draft_round(dc, nb, gamma, 0, 1, device="cuda")
    win, anchor, u = rd["window"], rd["anchor"].cuda(), rd["uniforms"].cuda()
    out = dd.buffers(nb, gamma)
    say("draft eager")
    dd.draft(win, anchor, u, 1.0, out)
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in out.items()}
    say("draft graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dd.draft(win, anchor, u, 1.0, out, stream=s)            # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dd.draft(win, anchor, u, 1.0, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for t in out.values():
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in out:
            assert torch.equal(out[n].view(torch.uint8), eager[n].view(torch.uint8)), f"replay {rep} {n}"
    # draft_logits rows are z plus the Markov row of the previous token
    B = dd.t["markov"]
    for b in range(nb):
        prev = int(anchor[b])
        for m in range(gamma):
            assert torch.equal(eager["draft_logits"][b, m], eager["z"][b, m] + B[prev])
            prev = int(eager["drafts"][b, m])
