"""Shared set-up for the GPU parity tests: seeded inputs on the device and the
matching fp64 oracle state, plus the comparison rules.

Comparison rules (floating point, written out here once):
  * fp32 results (f, s, windows, IIR state, fp32 outputs): normwise
    max|got - ref| <= 1e-5 * max|ref|  (elementwise relative error is
    undefined near zero).
  * bf16 outputs (y, o): elementwise |got - ref| <= 2e-2 + 2^-8 |ref|, and
    normwise max|got - ref| <= 2^-7 * max|ref| (a bf16 output is within
    2^-9 of its value, so this keeps a 4x margin while still catching a
    missing chunk of a long prefix).
  * integers (k, next token, best candidate, lengths) and copied bits
    (windows of bf16 inputs, KV rows): exact.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def f64(a) -> np.ndarray:
    return oracle.as_f64(a)


def assert_f32_close(got, ref, name, rel=1e-5):
    got, ref = f64(got), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= rel * max(scale, 1e-30), f"{name}: max|err| {err:.3e} > {rel} * {scale:.3e}"


def assert_bf16_close(got, ref, name):
    got, ref = f64(got), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if not got.size:
        return
    diff = np.abs(got - ref)
    bound = 2e-2 + 2.0 ** -8 * np.abs(ref)
    worst = int(np.argmax(diff - bound))
    assert np.all(diff <= bound), f"{name}: |err| {diff.flat[worst]:.3e} at {np.unravel_index(worst, diff.shape)}"
    scale = float(np.max(np.abs(ref)))
    assert float(diff.max()) <= 2.0 ** -7 * scale, f"{name}: normwise {diff.max():.3e} vs max|ref| {scale:.3e}"


def assert_out_close(cfg, got, ref, name):
    if cfg.act == synth.BF16:
        assert_bf16_close(got, ref, name)
    else:
        assert_f32_close(got, ref, name)


class Case:
    """One configuration set up on the GPU plus the matching oracle state."""

    def __init__(self, cfg, seed=0, needle=None, kv_cap=None, host_prefix=True, rnd=0, forced_len=None):
        self.cfg, self.seed = cfg, seed
        self.params = synth.make_layer(cfg, seed)
        self.small = synth.make_state_small(cfg, seed)
        self.tables = synth.make_tables(cfg, seed)
        self.anchor = synth.anchors(cfg, rnd, seed)
        self.ri = synth.round_inputs(cfg, self.anchor, rnd, seed, forced_len=forced_len)
        self.blk_np = synth.gather_block(cfg, self.tables, self.ri["tokens"])
        self.kv_cap = kv_cap or cfg.kv_cap()
        self.lay = dv.DeviceLayer(cfg, self.params)
        self.st = dv.DeviceState(self.lay, cfg.nb, self.kv_cap)
        self.st.load_small(self.small)
        self.prefix_host = []
        for b in range(cfg.nb):
            L = cfg.kv_lens[b]
            kp = synth.kv_prefix(cfg, b, "k", seed, device="cuda")
            vp = synth.kv_prefix(cfg, b, "v", seed, device="cuda")
            if needle:
                self._plant_needles(b, kp, needle)
            if L > 0:
                self.st.write_prefix(b, kp, vp)
            self.prefix_host.append((dv.to_host(kp), dv.to_host(vp)) if host_prefix else None)
            del kp, vp
        self.st.kv_len.copy_(torch.tensor(cfg.kv_lens, dtype=torch.int32))
        self.blk = dv.DeviceBlock(self.lay, cfg.nb, cfg.nc, cfg.gamma)
        self.blk.set_inputs(self.blk_np["x"], self.blk_np["q"], self.blk_np["k"], self.blk_np["v"])
        self.acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
        self.acc.set_inputs(self.ri["target_logits"], self.ri["drafts"], self.ri["draft_logits"], self.ri["uniforms"])
        torch.cuda.synchronize()

    def _plant_needles(self, b, kp, kind):
        """Scaled copies of block queries as keys, so that o is O(1) and masking is visible.

        prefix: for each block query i of candidate 0, key row pos_i := 4 q_i (positions
        seeded, plus the first and the last prefix row);  block keys: "self" sets
        k_j := 4 q_j (each query's own key dominates), "future" sets k_j := 4 q_{j-1}
        (a key that only a masking error would let query j-1 see).
        """
        cfg = self.cfg
        L = cfg.kv_lens[b]
        q = self.blk_np["q"]
        qb = torch.from_numpy(f64(q[b, 0]).astype(np.float32))          # [P][H][Dh]
        if L > 0:
            pos = list(synth.needle_positions(cfg, b, cfg.P, self.seed))
            pos[0], pos[-1] = 0, L - 1
            for i, p in enumerate(pos):
                kp[:, int(p), :] = (4.0 * qb[i]).to(kp.dtype).to(kp.device)
        k = self.blk_np["k"]
        q4 = q.copy()
        if cfg.act == synth.BF16:
            q4 = synth.bf16_bits(torch.from_numpy(4.0 * f64(q).astype(np.float32)))
        else:
            q4 = (4.0 * q).astype(np.float32)
        if kind == "self":
            k[b] = q4[b]
        elif kind == "future":
            k[b, :, 1:] = q4[b, :, :-1]

    # ------------------------------------------------------------ oracle side
    def oracle_state(self, b):
        kp, vp = self.prefix_host[b]
        return oracle.SeqState(self.small["short_win"][b], self.small["outer_win"][b], self.small["iir"][b],
                               [kp], [vp])

    def oracle_verify(self, b, c, heads=None):
        st = self.oracle_state(b)
        bn = self.blk_np
        x, q, k, v = bn["x"][b, c], bn["q"][b, c], bn["k"][b, c], bn["v"][b, c]
        if heads is not None:
            q, k, v = q[:, heads], k[:, heads], v[:, heads]
            st = oracle.SeqState(st.short_win, st.outer_win, st.iir,
                                 [blk[heads] for blk in st.k_blocks], [blk[heads] for blk in st.v_blocks])
        return oracle.verify_block(oracle.Layer.from_dict(self.params), st, x, q, k, v)

    def oracle_accept(self):
        cfg, ri = self.cfg, self.ri
        return oracle.accept_candidates(cfg.mode, ri["target_logits"], ri["draft_logits"], ri["drafts"],
                                        ri["uniforms"], cfg.temperature)

    # ------------------------------------------------------------ GPU side
    def run_verify(self):
        dv.verify(self.lay, self.st, self.blk, self.cfg.max_kv_len)

    def run_accept(self):
        mode = {"greedy": hci.GREEDY, "sample": hci.SAMPLE, "recursive": hci.SAMPLE_RECURSIVE}[self.cfg.mode]
        dv.accept(self.acc, mode, self.cfg.temperature)

    def run_slice(self):
        dv.slice_state(self.lay, self.st, self.blk, self.acc, self.cfg.max_kv_len)
