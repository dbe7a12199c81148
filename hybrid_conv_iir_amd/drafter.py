"""Device-side drafter: packed weights, the hci_drafter struct and the two calls."""
from __future__ import annotations

import ctypes

import torch

from . import hci
from .device import DEV


def _packed(w: torch.Tensor, device: str) -> torch.Tensor:
    w = w.to(device=device, dtype=torch.bfloat16).contiguous()
    wp = torch.empty(hci.linear_packed_elems(*w.shape), dtype=torch.bfloat16, device=device)
    hci.linear_pack(w, wp)
    return wp


class DeviceDrafter:
    def __init__(self, dc, params: dict, device: str = DEV):
        self.dc = dc
        f32 = lambda t: t.to(device=device, dtype=torch.float32).contiguous()
        self.t = {"w_proj": _packed(params["w_proj"], device),
                  "emb": params["emb"].to(device=device, dtype=torch.bfloat16).contiguous(),
                  "emb_t": _packed(params["emb"].t().contiguous(), device),
                  "mask": params["mask"].to(device=device, dtype=torch.bfloat16).contiguous(),
                  "g_f": f32(params["g_f"]), "markov": f32(params["markov"])}
        self.layer_t = []
        layers = (hci.DrafterLayer * dc.layers)()
        for l, p in enumerate(params["layers"]):
            t = {"g1": f32(p["g1"]), "g2": f32(p["g2"])}
            for n in ("w_qkv", "w_o", "w_up", "w_down"):
                t[n] = _packed(p[n], device)
            layers[l] = hci.DrafterLayer(t["g1"].data_ptr(), t["w_qkv"].data_ptr(), t["w_o"].data_ptr(),
                                         t["g2"].data_ptr(), t["w_up"].data_ptr(), t["w_down"].data_ptr())
            self.layer_t.append(t)
        self.layers = layers
        T = self.t
        self.c = hci.Drafter(dc.d_target, dc.d, dc.heads, dc.head_dim, dc.ffn, dc.vocab, dc.window, dc.layers, dc.eps,
                             T["w_proj"].data_ptr(), T["emb"].data_ptr(), T["emb_t"].data_ptr(), T["mask"].data_ptr(),
                             T["g_f"].data_ptr(), ctypes.cast(layers, ctypes.POINTER(hci.DrafterLayer)))
        self.ws = None

    def buffers(self, nb: int, gamma: int, device: str = DEV) -> dict:
        V = self.dc.vocab
        need = hci.draft_workspace_bytes(self.c, nb, gamma)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        return {"z": torch.empty((nb, gamma, V), dtype=torch.float32, device=device),
                "drafts": torch.empty((nb, gamma), dtype=torch.int32, device=device),
                "draft_logits": torch.empty((nb, gamma, V), dtype=torch.float32, device=device),
                "margin": torch.empty((nb, gamma), dtype=torch.float64, device=device)}

    def draft(self, window, anchor, uniforms, temperature: float, out: dict, stream=None) -> None:
        """Trunk pass then serial sampling; everything stays on the device."""
        nb, gamma = uniforms.shape
        hci.draft_logits(self.c, nb, gamma, window, anchor, out["z"], self.ws, stream)
        hci.draft_sample(nb, gamma, self.dc.vocab, temperature, out["z"], self.t["markov"], anchor, uniforms,
                         out["drafts"], out["draft_logits"], out["margin"], stream)
