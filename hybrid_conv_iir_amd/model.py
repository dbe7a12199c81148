"""Device-side buffers for a stack of full hybrid layers, and the calls on them.

Allocation with torch, then marshalling into the C ABI structs of
include/hci.h (hci_model, hci_model_state, hci_model_block); every step of
the verify and the slice runs in libhci's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List

import torch

from . import hci
from .device import DEV

_KIND = {"fir": hci.MIX_FIR, "iir": hci.MIX_IIR, "attn": hci.MIX_ATTN}


def _f32(t, device=DEV):
    return t.to(device=device, dtype=torch.float32).contiguous()


class DeviceModel:
    """Weights of every layer (projections packed once) and the hci_model struct."""

    def __init__(self, mc, params: List[Dict], device: str = DEV):
        self.mc = mc
        d = mc.d
        self.keep = []
        mixers = (hci.Mixer * len(params))()
        for l, p in enumerate(params):
            t = {"g": _f32(p["g"], device)}
            for name in ("w_in", "w_out"):
                w = p[name].to(device=device, dtype=torch.bfloat16).contiguous()
                K, N = w.shape
                wp = torch.empty(hci.linear_packed_elems(K, N), dtype=torch.bfloat16, device=device)
                hci.linear_pack(w, wp)
                t[name] = wp
            for name in ("w_short", "w_long", "lam", "beta", "c"):
                if name in p:
                    t[name] = _f32(p[name], device)
            ptr = lambda n: t[n].data_ptr() if n in t else None
            mixers[l] = hci.Mixer(_KIND[p["kind"]], mc.taps_short, mc.taps_long[l], mc.poles, ptr("g"), ptr("w_in"),
                                  ptr("w_out"), ptr("w_short"), ptr("w_long"), ptr("lam"), ptr("beta"), ptr("c"))
            self.keep.append(t)
        self.mixers = mixers
        self.c = hci.Model(len(params), d, mc.heads, mc.head_dim, mc.feature_layer, mc.feature_window, mc.eps,
                           ctypes.cast(mixers, ctypes.POINTER(hci.Mixer)))

    def attn_view(self):
        """An hci_layer describing one attention layer's cache geometry (for KV row access)."""
        mc = self.mc
        dummy = self.keep[0]["g"].data_ptr()
        return hci.Layer(mc.d, 1, 1, 1, mc.heads, mc.head_dim, hci.BF16, dummy, dummy, dummy, dummy, dummy)


class DeviceModelState:
    """Committed state of every layer for nb sequences, and the hci_model_state struct."""

    def __init__(self, model: DeviceModel, kv_cap: int, device: str = DEV):
        mc = self.mc = model.mc
        self.model, self.kv_cap = model, kv_cap
        d, nb = mc.d, mc.nb
        self.kv_len = torch.zeros(nb, dtype=torch.int32, device=device)
        self.feature = torch.zeros((nb, mc.feature_window, d), dtype=torch.bfloat16, device=device)
        self.layers = []
        states = (hci.LayerState * len(mc.kinds))()
        lv = model.attn_view()
        for l, kind in enumerate(mc.kinds):
            t = {}
            if kind == "attn":
                n = hci.kv_cache_elems(lv, nb, kv_cap)
                t["k_cache"] = torch.empty(n, dtype=torch.bfloat16, device=device)
                t["v_cache"] = torch.empty(n, dtype=torch.bfloat16, device=device)
            else:
                t["short_win"] = torch.zeros((nb, max(mc.taps_short - 1, 1), 3 * d), dtype=torch.float32, device=device)
                if kind == "fir":
                    t["long_win"] = torch.zeros((nb, max(mc.taps_long[l] - 1, 1), d), dtype=torch.float32,
                                                device=device)
                else:
                    t["iir"] = torch.zeros((nb, d, mc.poles), dtype=torch.float32, device=device)
            ptr = lambda n: t[n].data_ptr() if n in t else None
            states[l] = hci.LayerState(ptr("short_win"), ptr("long_win"), ptr("iir"), ptr("k_cache"), ptr("v_cache"))
            self.layers.append(t)
        self.states = states
        self.c = hci.ModelState(kv_cap, self.kv_len.data_ptr(), self.feature.data_ptr(),
                                ctypes.cast(states, ctypes.POINTER(hci.LayerState)))

    def _kv_state(self, l):
        t = self.layers[l]
        dummy = self.kv_len.data_ptr()
        return hci.State(self.kv_cap, dummy, dummy, dummy, t["k_cache"].data_ptr(), t["v_cache"].data_ptr(), dummy)

    def load(self, st: Dict) -> None:
        """Host or device tensors from synth.make_model_state."""
        mc = self.mc
        for l, kind in enumerate(mc.kinds):
            src, t = st["layers"][l], self.layers[l]
            if kind == "attn":
                for b in range(mc.nb):
                    k, v = src["k"][b].to(DEV).contiguous(), src["v"][b].to(DEV).contiguous()
                    if k.shape[1]:
                        hci.kv_write(self.model.attn_view(), self._kv_state(l), mc.nb, b, 0, k, v)
                continue
            if mc.taps_short > 1:
                t["short_win"].copy_(src["short_win"])
            if kind == "fir" and mc.taps_long[l] > 1:
                t["long_win"].copy_(src["long_win"])
            if kind == "iir":
                t["iir"].copy_(src["iir"])
        self.feature.copy_(st["feature"])
        self.kv_len.copy_(torch.tensor(mc.kv_lens, dtype=torch.int32))

    def kv_rows(self, l: int, b: int, row0: int, n: int):
        mc = self.mc
        k = torch.empty((mc.heads, n, mc.head_dim), dtype=torch.bfloat16, device=DEV)
        v = torch.empty_like(k)
        if n:
            hci.kv_read(self.model.attn_view(), self._kv_state(l), mc.nb, b, row0, k, v)
        return k, v

    def clone(self) -> "DeviceModelState":
        o = DeviceModelState(self.model, self.kv_cap)
        for a, b in zip(o.layers, self.layers):
            for n in a:
                a[n].copy_(b[n])
        o.feature.copy_(self.feature)
        o.kv_len.copy_(self.kv_len)
        return o


class DeviceModelBlock:
    """Block rows through every layer: x [L+1][rows][d] and each layer's retained z, u, s."""

    def __init__(self, model: DeviceModel, nb: int, nc: int, gamma: int, device: str = DEV):
        mc = model.mc
        self.model, self.nb, self.nc, self.gamma = model, nb, nc, gamma
        rows = self.rows = nb * nc * (gamma + 1)
        d = mc.d
        self.x = torch.zeros((len(mc.kinds) + 1, rows, d), dtype=torch.bfloat16, device=device)
        blocks = (hci.LayerBlock * len(mc.kinds))()
        self.layers = []
        for l, kind in enumerate(mc.kinds):
            t = {"z": torch.zeros((3, rows, d), dtype=torch.bfloat16 if kind == "attn" else torch.float32,
                                  device=device)}
            if kind == "fir":
                t["u"] = torch.zeros((rows, d), dtype=torch.float32, device=device)
            if kind == "iir":
                t["s"] = torch.zeros((rows, d, mc.poles), dtype=torch.float32, device=device)
            ptr = lambda n: t[n].data_ptr() if n in t else None
            blocks[l] = hci.LayerBlock(ptr("z"), ptr("u"), ptr("s"))
            self.layers.append(t)
        self.blocks = blocks
        self.c = hci.ModelBlock(self.x.data_ptr(), ctypes.cast(blocks, ctypes.POINTER(hci.LayerBlock)))
        self.ws = None

    def set_input(self, x_rows: torch.Tensor) -> None:
        self.x[0].copy_(x_rows)

    def ensure_workspace(self, max_kv_len: int) -> torch.Tensor:
        need = hci.model_workspace_bytes(self.model.c, self.nb, self.nc, self.gamma, max_kv_len)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.x.device)
        return self.ws


def verify(model: DeviceModel, st: DeviceModelState, blk: DeviceModelBlock, max_kv_len: int, stream=None) -> None:
    ws = blk.ensure_workspace(max_kv_len)
    hci.model_verify(model.c, st.c, blk.c, blk.nb, blk.nc, blk.gamma, max_kv_len, ws, stream)


def slice_state(model: DeviceModel, st: DeviceModelState, blk: DeviceModelBlock, max_kv_len: int, n_acc,
                best=None, stream=None) -> None:
    hci.model_slice(model.c, st.c, blk.c, blk.nb, blk.nc, blk.gamma, max_kv_len, n_acc,
                    best if blk.nc > 1 else None, stream)
