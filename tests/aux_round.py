"""A few verify -> accept -> slice rounds on the device, for the auxiliary checks.

Used in-process by tests/test_gpu_aux.py (checkpoint / resume, guard bands) and
as a child program (``python3 tests/aux_round.py OUT.npz``), plain and under
rocprofv3, for the instrumentation-neutrality check: the child writes every
output of every round and the final committed state as bit patterns.

Workload: two sequences of two candidate blocks (gamma = 6) of the d = 4096,
32 x 128-head layer, prefixes of 1000 and 777 tokens, sampling acceptance;
seeded synthetic inputs (hybrid_conv_iir_amd.synth), a new round of block
inputs and logits every round.  Product code only: no oracle.
"""
from __future__ import annotations

import os
import sys
from typing import Dict, Optional

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from hybrid_conv_iir_amd import device as dv  # noqa: E402
from hybrid_conv_iir_amd import hci, synth  # noqa: E402

ROUNDS = 4
SEED = 11


def config():
    return synth.scaled(synth.CONFIGS["mid8k"], kv_lens=(1000, 777), nc=2, gamma=6, vocab=384)


class Ctx:
    """Layer, tables and the initial state of the workload, on the device."""

    def __init__(self, seed: int = SEED):
        self.cfg = cfg = config()
        self.seed = seed
        self.params = synth.make_layer(cfg, seed)
        self.small = synth.make_state_small(cfg, seed)
        self.tables = synth.make_tables(cfg, seed)
        self.lay = dv.DeviceLayer(cfg, self.params)
        self.kv_cap = cfg.kv_cap(ROUNDS + 2)
        self.mode = hci.SAMPLE

    def new_state(self) -> dv.DeviceState:
        cfg = self.cfg
        st = dv.DeviceState(self.lay, cfg.nb, self.kv_cap)
        st.load_small(self.small)
        for b in range(cfg.nb):
            st.write_prefix(b, synth.kv_prefix(cfg, b, "k", self.seed, device="cuda"),
                            synth.kv_prefix(cfg, b, "v", self.seed, device="cuda"))
        st.kv_len.copy_(torch.tensor(cfg.kv_lens, dtype=torch.int32))
        return st

    def round_data(self, rnd: int):
        cfg = self.cfg
        anchor = synth.anchors(cfg, rnd, self.seed)
        ri = synth.round_inputs(cfg, anchor, rnd, self.seed)
        bn = synth.gather_block(cfg, self.tables, ri["tokens"])
        return ri, bn


def run_rounds(ctx: Ctx, st: dv.DeviceState, r0: int, r1: int,
               blk: Optional[dv.DeviceBlock] = None, acc: Optional[dv.DeviceAccept] = None,
               bound0: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Rounds r0 .. r1 - 1 on state st; the outputs of every round, stacked, as host arrays."""
    cfg = ctx.cfg
    blk = blk or dv.DeviceBlock(ctx.lay, cfg.nb, cfg.nc, cfg.gamma)
    acc = acc or dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    bound = ctx.kv_cap - cfg.P if bound0 is None else bound0
    out: Dict[str, list] = {k: [] for k in ("f", "s", "y", "o", "n_acc", "next", "best", "margin")}
    for rnd in range(r0, r1):
        ri, bn = ctx.round_data(rnd)
        blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
        acc.set_inputs(ri["target_logits"], ri["drafts"], ri["draft_logits"], ri["uniforms"])
        dv.verify(ctx.lay, st, blk, bound)
        dv.accept(acc, ctx.mode, cfg.temperature, status=st.status)
        dv.slice_state(ctx.lay, st, blk, acc, bound)
        for name in ("f", "s", "y", "o"):
            out[name].append(dv.to_host(getattr(blk, name)))
        for name in ("n_acc", "next", "best", "margin"):
            out[name].append(dv.to_host(getattr(acc, name)))
    torch.cuda.synchronize()
    return {k: np.stack(v) for k, v in out.items() if v}


def snapshot(ctx: Ctx, st: dv.DeviceState) -> Dict[str, np.ndarray]:
    """The committed state as host arrays, bit for bit: windows, IIR state, lengths, status words
    and the committed KV rows of every sequence (read through the library's row interface)."""
    snap = {"short_win": dv.to_host(st.short_win), "outer_win": dv.to_host(st.outer_win),
            "iir": dv.to_host(st.iir), "kv_len": dv.to_host(st.kv_len), "status": dv.to_host(st.status)}
    for b in range(ctx.cfg.nb):
        L = int(snap["kv_len"][b])
        k, v = st.read_rows(b, 0, L)
        snap[f"k{b}"], snap[f"v{b}"] = dv.to_host(k), dv.to_host(v)
    return snap


def restore(ctx: Ctx, snap: Dict[str, np.ndarray]) -> dv.DeviceState:
    """A fresh device state holding exactly the snapshot."""
    st = dv.DeviceState(ctx.lay, ctx.cfg.nb, ctx.kv_cap)
    st.short_win.copy_(dv.to_dev(snap["short_win"]))
    st.outer_win.copy_(dv.to_dev(snap["outer_win"]))
    st.iir.copy_(dv.to_dev(snap["iir"]))
    for b in range(ctx.cfg.nb):
        if snap[f"k{b}"].shape[1] > 0:
            st.write_prefix(b, dv.to_dev(snap[f"k{b}"]), dv.to_dev(snap[f"v{b}"]))
    st.kv_len.copy_(dv.to_dev(snap["kv_len"]))
    st.status.copy_(dv.to_dev(snap["status"]))
    torch.cuda.synchronize()
    return st


def full_run(ctx: Ctx) -> Dict[str, np.ndarray]:
    st = ctx.new_state()
    out = run_rounds(ctx, st, 0, ROUNDS)
    out.update({"state_" + k: v for k, v in snapshot(ctx, st).items()})
    return out


def main() -> int:
    path = sys.argv[1]
    out = full_run(Ctx())
    np.savez(path, **out)
    print("AUX_ROUND_DONE", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
