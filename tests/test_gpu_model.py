"""GPU stack of full hybrid layers (Hyena FIR / IIR mixers, attention, projections, norms)
against the fp64 oracle with the same bf16 rounding points.

Tolerance (derived from the arithmetic): both sides round a, y and the new
residual stream x to bf16 -- the device from fp32 sums, the oracle from fp64
ones -- so a value within the sums' difference of a bf16 midpoint rounds to
the neighbouring bf16 on one side (one ulp, 2^-8..2^-7 of the value).  Each
such difference moves every output of the next projection a little, which
makes more rounding decisions differ downstream: layer by layer the two
residual streams decorrelate at the level of a few ulps of their typical
magnitude (not of each element).  Every tensor, bf16 or fp32, is therefore
held elementwise to 2^-5 rms(ref) + 2^-6 |ref| -- about eight bf16 ulps at
typical magnitude -- while an indexing or arithmetic mistake moves values by
O(rms).  Layer 0 sees identical inputs on both sides (the block rows x0): there
the only differences are the fp32 sums and a few bf16 rounding decisions of a,
so its tensors are held eight times tighter, 2^-8 rms(ref) + 2^-9 |ref| for fp32
and 2^-8 rms(ref) + 2^-7 |ref| (one bf16 ulp) for the bf16 residual stream x[1].
That catches small systematic errors the stack-wide bound lets through: in the
oracle, leaving out the bf16 rounding of a moves layer-0 z by 0.0058 rms (the
stack bound is 2^-5 = 0.031 rms, the layer-0 bound 2^-8 = 0.0039 rms).
"""
import numpy as np
import pytest
import torch

from oracle import model as OM
from hybrid_conv_iir_amd import model as dm
from hybrid_conv_iir_amd import synth
from gpu_harness import say

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def oracle_model(mc, params):
    mixers = []
    for p in params:
        mx = OM.Mixer(kind=p["kind"], g=f64(p["g"]), w_in=f64(p["w_in"]), w_out=f64(p["w_out"]))
        for name, attr in (("w_short", "w_short"), ("w_long", "w_long"), ("lam", "lam"), ("beta", "beta"), ("c", "c")):
            if name in p:
                setattr(mx, attr, f64(p[name]))
        mixers.append(mx)
    return OM.Model(mixers, mc.d, mc.heads, mc.head_dim, mc.eps, mc.feature_layer, mc.feature_window)


def oracle_state(mc, st, b):
    layers = []
    for l, kind in enumerate(mc.kinds):
        src = st["layers"][l]
        if kind == "attn":
            layers.append(OM.LayerState(k_blocks=[f64(src["k"][b])], v_blocks=[f64(src["v"][b])]))
            continue
        ls = OM.LayerState(short_win=f64(src["short_win"][b]))
        if kind == "fir":
            ls.long_win = f64(src["long_win"][b])
        else:
            ls.iir = f64(src["iir"][b])
        layers.append(ls)
    return OM.ModelState(layers, f64(st["feature"][b]))


def close(got, ref, tag):
    got, ref = f64(got), np.asarray(ref, np.float64)
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-30)
    err = np.abs(got - ref)
    ok = err <= 2.0 ** -5 * rms + 2.0 ** -6 * np.abs(ref)
    assert ok.all(), f"{tag}: {int((~ok).sum())} of {ok.size} outside, max err / rms {err.max() / rms:.3g}"
    return err.max() / rms


close_bf16 = close_f32 = close


def close_l0(got, ref, tag, ulp_rel):
    """the layer-0 bound: 2^-8 rms(ref) + ulp_rel |ref|"""
    got, ref = f64(got), np.asarray(ref, np.float64)
    rms = max(float(np.sqrt(np.mean(ref * ref))), 1e-30)
    err = np.abs(got - ref)
    ok = err <= 2.0 ** -8 * rms + ulp_rel * np.abs(ref)
    assert ok.all(), f"{tag}: {int((~ok).sum())} of {ok.size} outside the layer-0 bound, max err / rms {err.max() / rms:.3g}"


def close_product(got, ref, f1, f2, tag):
    """u = f1 * f2 of two factors each held to the bound above: the product rule carries it over as
    2^-5 (rms(f1) |f2| + rms(f2) |f1|) + 2^-6 |u|."""
    got, ref = f64(got), np.asarray(ref, np.float64)
    r1, r2 = (max(float(np.sqrt(np.mean(f * f))), 1e-30) for f in (f1, f2))
    bound = 2.0 ** -5 * (r1 * np.abs(f2) + r2 * np.abs(f1)) + 2.0 ** -6 * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    ok = err <= bound
    assert ok.all(), f"{tag}: {int((~ok).sum())} of {ok.size} outside, max err / bound {np.max(err / bound):.3g}"


class ModelCase:
    def __init__(self, mc, seed=0, extra_cap=64):
        self.mc = mc
        self.params = synth.make_model(mc, seed, device="cuda")
        self.st_host = synth.make_model_state(mc, seed, device="cuda")
        self.dmodel = dm.DeviceModel(mc, self.params)
        cap = (max(mc.kv_lens) + extra_cap + 31) // 32 * 32
        self.st = dm.DeviceModelState(self.dmodel, cap)
        self.st.load(self.st_host)
        self.blk = dm.DeviceModelBlock(self.dmodel, mc.nb, mc.nc, mc.gamma)
        self.x0 = synth.model_block_input(mc, 0, seed, device="cuda")
        self.blk.set_input(self.x0)
        self.om = oracle_model(mc, self.params)

    def rows(self, b, c):
        r0 = (b * self.mc.nc + c) * self.mc.P
        return slice(r0, r0 + self.mc.P)


def _check_verify_and_slice(case: ModelCase, ks, best=None):
    mc = case.mc
    say(f"model {mc.name} d={mc.d} kinds={mc.kinds} nb={mc.nb} nc={mc.nc} gamma={mc.gamma} L={mc.kv_lens}")
    dm.verify(case.dmodel, case.st, case.blk, max(mc.kv_lens))
    torch.cuda.synchronize()
    fwds = {}
    for b in range(mc.nb):
        ost = oracle_state(mc, case.st_host, b)
        for c in range(mc.nc):
            rs = case.rows(b, c)
            fwd = OM.model_verify_block(case.om, ost, f64(case.x0[rs]), rounding=True)
            fwds[b, c] = (ost, fwd)
            tag = f"{mc.name}[b{b},c{c}]"
            rec0, lb0 = fwd["layers"][0], case.blk.layers[0]
            close_l0(case.blk.x[1][rs], fwd["x"][1], f"{tag} x[1]", 2.0 ** -7)
            close_l0(lb0["z"][:, rs], rec0["z"], f"{tag} layer 0 z", 2.0 ** -9)
            if "s" in rec0:
                close_l0(lb0["s"][rs], rec0["s"], f"{tag} layer 0 s", 2.0 ** -9)
            for l in range(len(mc.kinds)):
                close_bf16(case.blk.x[l + 1][rs], fwd["x"][l + 1], f"{tag} x[{l + 1}]")
                rec, lb = fwd["layers"][l], case.blk.layers[l]
                close_f32(lb["z"][:, rs], rec["z"], f"{tag} layer {l} z")
                if "u" in rec:
                    close_product(lb["u"][rs], rec["u"], rec["zh"][1], rec["zh"][2], f"{tag} layer {l} u")
                if "s" in rec:
                    close_f32(lb["s"][rs], rec["s"], f"{tag} layer {l} s")
    say(f"model {mc.name} slice k={ks}")
    n_acc = torch.zeros((mc.nb, mc.nc), dtype=torch.int32, device="cuda")
    bc = torch.zeros(mc.nb, dtype=torch.int32, device="cuda")
    for b in range(mc.nb):
        cs = 0 if best is None else best[b]
        n_acc[b, cs] = ks[b]
        bc[b] = cs
    dm.slice_state(case.dmodel, case.st, case.blk, max(mc.kv_lens), n_acc, bc)
    torch.cuda.synchronize()
    for b in range(mc.nb):
        cs = 0 if best is None else best[b]
        ost, fwd = fwds[b, cs]
        new = OM.model_slice_state(case.om, ost, fwd, ks[b])
        tag = f"{mc.name}[b{b}] slice k={ks[b]} c*={cs}"
        assert int(case.st.kv_len[b]) == mc.kv_lens[b] + ks[b] + 1, tag
        close_bf16(case.st.feature[b], new.feature, tag + " feature")
        for l, kind in enumerate(mc.kinds):
            t, nl = case.st.layers[l], new.layers[l]
            if kind == "attn":
                L = mc.kv_lens[b]
                kr, vr = case.st.kv_rows(l, b, L, ks[b] + 1)
                close_bf16(kr, nl.k_blocks[-1], f"{tag} layer {l} k rows")
                close_bf16(vr, nl.v_blocks[-1], f"{tag} layer {l} v rows")
                k0, _ = case.st.kv_rows(l, b, 0, L)          # committed rows untouched
                np.testing.assert_array_equal(f64(k0), f64(case.st_host["layers"][l]["k"][b]))
                continue
            if mc.taps_short > 1:
                close_f32(t["short_win"][b], nl.short_win, f"{tag} layer {l} short_win")
            if kind == "fir" and mc.taps_long[l] > 1:
                # the window's newest rows are u values (products), the rest were committed before
                Wl = mc.taps_long[l] - 1
                newer = min(ks[b] + 1, Wl)
                zh = fwd["layers"][l]["zh"][:, : ks[b] + 1][:, -newer:]
                close_product(t["long_win"][b][Wl - newer:], nl.long_win[Wl - newer:], zh[1], zh[2],
                              f"{tag} layer {l} long_win (new rows)")
                np.testing.assert_array_equal(f64(t["long_win"][b][: Wl - newer]), nl.long_win[: Wl - newer])
            if kind == "iir":
                close_f32(t["iir"][b], nl.iir, f"{tag} layer {l} iir")


def test_model_stack_small():
    case = ModelCase(synth.MODEL_CONFIGS["m4_small"])
    _check_verify_and_slice(case, ks=[3, 6])


def test_model_stack_two_attention_layers_k0():
    mc = synth.model_scaled(synth.MODEL_CONFIGS["m4_small"], kinds=("attn", "iir", "fir", "attn"),
                            taps_long=(0, 0, 33, 0), feature_layer=0, feature_window=3, kv_lens=(0, 65, 31),
                            gamma=12, cfg_id=211)
    _check_verify_and_slice(ModelCase(mc), ks=[0, 12, 5])


def test_model_stack_multi_candidate():
    mc = synth.model_scaled(synth.MODEL_CONFIGS["m4_small"], nc=3, gamma=5, kv_lens=(129, 1), cfg_id=212)
    _check_verify_and_slice(ModelCase(mc), ks=[2, 5], best=[2, 1])


def test_model_stack_full_width():
    """d = 4096, 32 heads of 128, the 4-layer stripe over a 4096-token prefix."""
    mc = synth.model_scaled(synth.MODEL_CONFIGS["m4_long"], kv_lens=(4096,), cfg_id=213)
    _check_verify_and_slice(ModelCase(mc), ks=[7])


def test_model_block_plus_slice_matches_sequential_steps_on_gpu():
    """verify(gamma) + slice(k) against k+1 one-row verifies + slices, for every k (device only)."""
    mc = synth.model_scaled(synth.MODEL_CONFIGS["m4_small"], kv_lens=(77,), gamma=5, cfg_id=214)
    base = ModelCase(mc)
    dm.verify(base.dmodel, base.st, base.blk, mc.kv_lens[0])
    torch.cuda.synchronize()
    one = synth.model_scaled(mc, gamma=0)
    blk1 = dm.DeviceModelBlock(base.dmodel, 1, 1, 0)
    zero = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    for k in range(mc.P):
        say(f"model contract k={k}")
        a = base.st.clone()
        dm.slice_state(base.dmodel, a, base.blk, mc.kv_lens[0], torch.full((1, 1), k, dtype=torch.int32,
                                                                            device="cuda"))
        s = base.st.clone()
        outs = []
        for i in range(k + 1):
            blk1.set_input(base.x0[i: i + 1])
            dm.verify(base.dmodel, s, blk1, mc.kv_lens[0] + i)
            dm.slice_state(base.dmodel, s, blk1, mc.kv_lens[0] + i, zero)
            outs.append(blk1.x[-1, 0].clone())
        torch.cuda.synchronize()
        assert int(a.kv_len[0]) == int(s.kv_len[0]) == mc.kv_lens[0] + k + 1
        close_bf16(torch.stack(outs), f64(base.blk.x[-1][: k + 1]), f"k={k} outputs")
        close_bf16(a.feature, f64(s.feature), f"k={k} feature")
        for l, kind in enumerate(mc.kinds):
            if kind == "attn":
                ka, va = a.kv_rows(l, 0, 0, mc.kv_lens[0] + k + 1)
                kb, vb = s.kv_rows(l, 0, 0, mc.kv_lens[0] + k + 1)
                close_bf16(ka, f64(kb), f"k={k} layer {l} k")
                close_bf16(va, f64(vb), f"k={k} layer {l} v")
                continue
            for n in a.layers[l]:
                close_f32(a.layers[l][n], f64(s.layers[l][n]), f"k={k} layer {l} {n}")


def test_model_stack_graph_replay_equals_eager():
    """The stack verify captured in a HIP graph replays to the eager call's bits: every layer's
    tensors and the residual stream (no memset is recorded; the workspace is allocated before the
    capture).  The outputs are cleared by eager work before each replay."""
    mc = synth.model_scaled(synth.MODEL_CONFIGS["m4_small"], nc=2, gamma=5, kv_lens=(129, 40), cfg_id=215)
    case = ModelCase(mc)
    bound = max(mc.kv_lens)
    outs = [case.blk.x] + [t for lb in case.blk.layers for t in lb.values() if isinstance(t, torch.Tensor)]
    say("model graph: eager verify")
    dm.verify(case.dmodel, case.st, case.blk, bound)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    x0 = case.blk.x[0].clone()
    say("model graph: capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dm.verify(case.dmodel, case.st, case.blk, bound, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        case.blk.x[0].copy_(x0)
        torch.cuda.synchronize()
        say(f"model graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), f"replay {rep}: output tensor {i}"
