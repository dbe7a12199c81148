"""Device-side buffers for one layer: allocation and host<->device copies.

Plumbing around the C ABI: torch supplies device memory and streams, this
module sizes the buffers the way include/hci.h lays them out and hands the
pointers to ``hci``.  No step of the method runs here.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import hci

DEV = "cuda"


def to_dev(a: np.ndarray, act: Optional[int] = None, device: str = DEV) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceLayer:
    def __init__(self, cfg, params: Dict[str, np.ndarray], device: str = DEV):
        self.cfg = cfg
        self.act = hci.BF16 if cfg.act == "bf16" else hci.F32
        self.t = {k: to_dev(np.asarray(v, np.float32), device=device) for k, v in params.items()}
        self.c = hci.make_layer(cfg.d, cfg.taps_short, cfg.taps_outer, cfg.poles, cfg.heads, cfg.head_dim,
                                self.act, self.t["w_short"], self.t["w_outer"], self.t["lam"], self.t["beta"],
                                self.t["c"])


class DeviceState:
    """Committed state of nb sequences (windows, IIR, tiled KV cache, lengths)."""

    def __init__(self, layer: DeviceLayer, nb: int, kv_cap: int, device: str = DEV):
        cfg = layer.cfg
        self.layer, self.nb, self.kv_cap = layer, nb, kv_cap
        at = hci.act_torch_dtype(layer.act)
        self.short_win = torch.zeros((nb, max(cfg.taps_short - 1, 1), cfg.d), dtype=at, device=device)
        self.outer_win = torch.zeros((nb, max(cfg.taps_outer - 1, 1), cfg.d), dtype=torch.float32, device=device)
        self.iir = torch.zeros((nb, cfg.d, cfg.poles), dtype=torch.float32, device=device)
        n = hci.kv_cache_elems(layer.c, nb, kv_cap)
        if n == 0:
            raise ValueError("invalid cache geometry")
        self.k_cache = torch.empty(n, dtype=at, device=device)
        self.v_cache = torch.empty(n, dtype=at, device=device)
        self.kv_len = torch.zeros(nb, dtype=torch.int32, device=device)
        self.status = torch.zeros(nb, dtype=torch.int32, device=device)     # HCI_DS_* bits per sequence
        self.c = hci.make_state(layer.act, kv_cap, self.short_win, self.outer_win, self.iir,
                                self.k_cache, self.v_cache, self.kv_len, self.status)

    def load_small(self, st: Dict[str, np.ndarray]) -> None:
        cfg = self.layer.cfg
        if cfg.taps_short > 1:
            self.short_win.copy_(to_dev(st["short_win"]))
        if cfg.taps_outer > 1:
            self.outer_win.copy_(to_dev(st["outer_win"]))
        self.iir.copy_(to_dev(st["iir"]))

    def write_prefix(self, b: int, k_rows: torch.Tensor, v_rows: torch.Tensor, row0: int = 0) -> None:
        """k_rows, v_rows: device [H][n][Dh] act."""
        hci.kv_write(self.layer.c, self.c, self.nb, b, row0, k_rows.contiguous(), v_rows.contiguous())

    def read_rows(self, b: int, row0: int, n: int):
        cfg = self.layer.cfg
        at = hci.act_torch_dtype(self.layer.act)
        k = torch.empty((cfg.heads, n, cfg.head_dim), dtype=at, device=self.k_cache.device)
        v = torch.empty_like(k)
        if n > 0:
            hci.kv_read(self.layer.c, self.c, self.nb, b, row0, k, v)
        return k, v

    def snapshot(self) -> Dict[str, np.ndarray]:
        cfg = self.layer.cfg
        out = {"iir": to_host(self.iir), "kv_len": to_host(self.kv_len)}
        out["short_win"] = to_host(self.short_win)[:, : cfg.taps_short - 1]
        out["outer_win"] = to_host(self.outer_win)[:, : cfg.taps_outer - 1]
        return out


class DeviceBlock:
    """Block inputs, retained intermediates and outputs for nb x nc blocks of P positions."""

    def __init__(self, layer: DeviceLayer, nb: int, nc: int, gamma: int, device: str = DEV):
        cfg = layer.cfg
        self.layer, self.nb, self.nc, self.gamma = layer, nb, nc, gamma
        P = gamma + 1
        at = hci.act_torch_dtype(layer.act)
        H, Dh, d = cfg.heads, cfg.head_dim, cfg.d
        self.x = torch.zeros((nb, nc, P, d), dtype=at, device=device)
        self.q = torch.zeros((nb, nc, P, H, Dh), dtype=at, device=device)
        self.k = torch.zeros_like(self.q)
        self.v = torch.zeros_like(self.q)
        self.f = torch.zeros((nb, nc, P, d), dtype=torch.float32, device=device)
        self.s = torch.zeros((nb, nc, P, d, cfg.poles), dtype=torch.float32, device=device)
        self.y = torch.zeros((nb, nc, P, d), dtype=at, device=device)
        self.o = torch.zeros((nb, nc, P, H, Dh), dtype=at, device=device)
        self.c = hci.make_block(layer.act, self.x, self.q, self.k, self.v, self.f, self.s, self.y, self.o)
        self.ws = None

    def set_inputs(self, x, q, k, v) -> None:
        for dst, src in ((self.x, x), (self.q, q), (self.k, k), (self.v, v)):
            dst.copy_(src if isinstance(src, torch.Tensor) else to_dev(src))

    def ensure_workspace(self, max_kv_len: int) -> torch.Tensor:
        need = hci.verify_workspace_bytes(self.layer.c, self.nb, self.nc, self.gamma, max_kv_len)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.x.device)
        return self.ws


class DeviceTree:
    """A token tree of n nodes per sequence: parents, per-node inputs, retained intermediates and
    outputs, plus the acceptance buffers of its walk."""

    def __init__(self, layer: DeviceLayer, nb: int, n: int, vocab: int = 1, device: str = DEV):
        cfg = layer.cfg
        self.layer, self.nb, self.n, self.vocab = layer, nb, n, vocab
        at = hci.act_torch_dtype(layer.act)
        H, Dh, d = cfg.heads, cfg.head_dim, cfg.d
        self.parent = torch.full((nb, n), -1, dtype=torch.int32, device=device)
        self.x = torch.zeros((nb, n, d), dtype=at, device=device)
        self.q = torch.zeros((nb, n, H, Dh), dtype=at, device=device)
        self.k = torch.zeros_like(self.q)
        self.v = torch.zeros_like(self.q)
        self.f = torch.zeros((nb, n, d), dtype=torch.float32, device=device)
        self.s = torch.zeros((nb, n, d, cfg.poles), dtype=torch.float32, device=device)
        self.y = torch.zeros((nb, n, d), dtype=at, device=device)
        self.o = torch.zeros((nb, n, H, Dh), dtype=at, device=device)
        self.tokens = torch.zeros((nb, n), dtype=torch.int32, device=device)
        self.zt = torch.zeros((nb, n, vocab), dtype=torch.float32, device=device)
        self.zd = torch.zeros((nb, n, vocab), dtype=torch.float32, device=device)
        self.u = torch.zeros((nb, n), dtype=torch.float64, device=device)
        self.n_acc = torch.zeros(nb, dtype=torch.int32, device=device)
        self.path = torch.zeros((nb, n), dtype=torch.int32, device=device)
        self.next = torch.zeros(nb, dtype=torch.int32, device=device)
        self.margin = torch.zeros(nb, dtype=torch.float64, device=device)
        self.c = hci.make_tree(layer.act, self.parent, self.x, self.q, self.k, self.v, self.f, self.s, self.y, self.o)
        self.ws = None

    def set_inputs(self, parent, x, q, k, v) -> None:
        for dst, src in ((self.parent, parent), (self.x, x), (self.q, q), (self.k, k), (self.v, v)):
            dst.copy_(src if isinstance(src, torch.Tensor) else to_dev(np.ascontiguousarray(src)))

    def set_accept_inputs(self, tokens, zt, zd=None, u=None) -> None:
        self.tokens.copy_(to_dev(np.asarray(tokens, np.int32)))
        self.zt.copy_(to_dev(np.asarray(zt, np.float32)))
        if zd is not None:
            self.zd.copy_(to_dev(np.asarray(zd, np.float32)))
        if u is not None:
            self.u.copy_(to_dev(np.asarray(u, np.float64)))

    def ensure_workspace(self, max_kv_len: int) -> torch.Tensor:
        need = hci.verify_workspace_bytes(self.layer.c, self.nb, 1, self.n - 1, max_kv_len)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.x.device)
        return self.ws


def verify_tree(layer: DeviceLayer, state: "DeviceState", tree: DeviceTree, max_kv_len: int, stream=None) -> None:
    ws = tree.ensure_workspace(max_kv_len)
    hci.verify_tree(layer.c, state.c, tree.c, tree.nb, tree.n, max_kv_len, ws, stream)


def accept_tree(tree: DeviceTree, mode: int, temperature: float = 1.0, stream=None, status=None) -> None:
    sample = mode != hci.GREEDY
    hci.accept_tree(mode, tree.nb, tree.n, tree.vocab, temperature, tree.parent, tree.tokens, tree.zt,
                    tree.zd if sample else None, tree.u if sample else None, tree.n_acc, tree.path, tree.next,
                    tree.margin, status, stream)


def slice_tree(layer: DeviceLayer, state: "DeviceState", tree: DeviceTree, max_kv_len: int, stream=None) -> None:
    hci.slice_tree(layer.c, state.c, tree.c, tree.nb, tree.n, max_kv_len, tree.n_acc, tree.path, stream)


class DeviceAccept:
    """Acceptance inputs and outputs for nb x nc blocks."""

    def __init__(self, nb: int, nc: int, gamma: int, vocab: int, device: str = DEV):
        P = gamma + 1
        self.nb, self.nc, self.gamma, self.vocab = nb, nc, gamma, vocab
        self.zt = torch.zeros((nb, nc, P, vocab), dtype=torch.float32, device=device)
        self.zd = torch.zeros((nb, nc, max(gamma, 1), vocab), dtype=torch.float32, device=device)
        self.drafts = torch.zeros((nb, nc, max(gamma, 1)), dtype=torch.int32, device=device)
        self.u = torch.zeros((nb, nc, P), dtype=torch.float64, device=device)
        self.n_acc = torch.zeros((nb, nc), dtype=torch.int32, device=device)
        self.next = torch.zeros((nb, nc), dtype=torch.int32, device=device)
        self.best = torch.zeros(nb, dtype=torch.int32, device=device)
        self.margin = torch.zeros((nb, nc), dtype=torch.float64, device=device)

    def set_inputs(self, zt, drafts, zd=None, u=None) -> None:
        self.zt.copy_(to_dev(np.asarray(zt, np.float32)))
        if self.gamma > 0:
            self.drafts.copy_(to_dev(np.asarray(drafts, np.int32)))
        if zd is not None and self.gamma > 0:
            self.zd.copy_(to_dev(np.asarray(zd, np.float32)))
        if u is not None:
            self.u.copy_(to_dev(np.asarray(u, np.float64)))


def verify(layer: DeviceLayer, state: DeviceState, blk: DeviceBlock, max_kv_len: int, stream=None) -> None:
    ws = blk.ensure_workspace(max_kv_len)
    hci.verify_block(layer.c, state.c, blk.c, blk.nb, blk.nc, blk.gamma, max_kv_len, ws, stream)


def accept(acc: DeviceAccept, mode: int, temperature: float = 1.0, stream=None, status=None) -> None:
    """status: the [nb] status words to report into (e.g. DeviceState.status), or None."""
    sample = mode != hci.GREEDY
    hci.accept(mode, acc.nb, acc.nc, acc.gamma, acc.vocab, temperature, acc.zt,
               acc.zd if sample else None, acc.drafts, acc.u if sample else None,
               acc.n_acc, acc.next, acc.best, acc.margin, stream, status)


def slice_state(layer: DeviceLayer, state: DeviceState, blk: DeviceBlock, acc: DeviceAccept, max_kv_len: int,
                stream=None) -> None:
    hci.slice_state(layer.c, state.c, blk.c, blk.nb, blk.nc, blk.gamma, max_kv_len, acc.n_acc,
                    acc.best if blk.nc > 1 else None, stream)
