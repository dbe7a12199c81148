"""Python binding of libhci (ctypes): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
their dtype / shape / contiguity against the C ABI (include/hci.h), and
passes raw pointers and the current HIP stream.  All arithmetic happens in
the HIP kernels; if the library is missing this module raises on import.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhci.so")

OK, EINVAL, ECAPACITY, EUNSUPPORTED, EDEVICE, EWORKSPACE = 0, -1, -2, -3, -4, -5
# device status bits (include/hci.h, HCI_DS_*)
DS_NONFINITE, DS_K_RANGE, DS_CAND_RANGE, DS_KV_LEN, DS_DRAFT_ID, DS_TREE = 0x1, 0x2, 0x4, 0x8, 0x10, 0x20
F32, BF16 = 0, 1
GREEDY, SAMPLE, SAMPLE_RECURSIVE = 0, 1, 2
KV_TILE = 32


class HciError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libhci.so not built at {LIB_PATH}; run `python -m hybrid_conv_iir_amd.build`")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class Layer(ctypes.Structure):
    _fields_ = [("d", _i), ("taps_short", _i), ("taps_outer", _i), ("poles", _i), ("heads", _i),
                ("head_dim", _i), ("act_dtype", _i), ("w_short", _p), ("w_outer", _p), ("lambda_", _p),
                ("beta", _p), ("c", _p)]


class State(ctypes.Structure):
    _fields_ = [("kv_cap", _i), ("short_win", _p), ("outer_win", _p), ("iir", _p), ("k_cache", _p),
                ("v_cache", _p), ("kv_len", _p), ("status", _p)]


class Block(ctypes.Structure):
    _fields_ = [("x", _p), ("q", _p), ("k", _p), ("v", _p), ("f", _p), ("s", _p), ("y", _p), ("o", _p)]


class Tree(ctypes.Structure):
    _fields_ = [("parent", _p), ("x", _p), ("q", _p), ("k", _p), ("v", _p), ("f", _p), ("s", _p), ("y", _p),
                ("o", _p)]


MIX_FIR, MIX_IIR, MIX_ATTN = 0, 1, 2


class Mixer(ctypes.Structure):
    _fields_ = [("kind", _i), ("taps_short", _i), ("taps_long", _i), ("poles", _i), ("norm", _p), ("w_in", _p),
                ("w_out", _p), ("w_short", _p), ("w_long", _p), ("lambda_", _p), ("beta", _p), ("c", _p)]


class Model(ctypes.Structure):
    _fields_ = [("n_layers", _i), ("d", _i), ("heads", _i), ("head_dim", _i), ("feature_layer", _i),
                ("feature_window", _i), ("eps", ctypes.c_float), ("layers", ctypes.POINTER(Mixer))]


class LayerState(ctypes.Structure):
    _fields_ = [("short_win", _p), ("long_win", _p), ("iir", _p), ("k_cache", _p), ("v_cache", _p)]


class ModelState(ctypes.Structure):
    _fields_ = [("kv_cap", _i), ("kv_len", _p), ("feature", _p), ("layers", ctypes.POINTER(LayerState))]


class LayerBlock(ctypes.Structure):
    _fields_ = [("z", _p), ("u", _p), ("s", _p)]


class ModelBlock(ctypes.Structure):
    _fields_ = [("x", _p), ("layers", ctypes.POINTER(LayerBlock))]


class DrafterLayer(ctypes.Structure):
    _fields_ = [("g1", _p), ("w_qkv", _p), ("w_o", _p), ("g2", _p), ("w_up", _p), ("w_down", _p)]


class Drafter(ctypes.Structure):
    _fields_ = [("d_target", _i), ("d", _i), ("heads", _i), ("head_dim", _i), ("ffn", _i), ("vocab", _i),
                ("window", _i), ("n_layers", _i), ("eps", ctypes.c_float), ("w_proj", _p), ("emb", _p),
                ("emb_t", _p), ("mask", _p), ("g_f", _p), ("layers", ctypes.POINTER(DrafterLayer))]


EXPORTS = {
    "hci_status_string": (_i, [_i, ctypes.c_char_p, _sz]),
    "hci_device_status_string": (_i, [ctypes.c_uint32, ctypes.c_char_p, _sz]),
    "hci_version": (_i, []),
    "hci_verify_workspace_bytes": (_sz, [ctypes.POINTER(Layer), _i, _i, _i, _i]),
    "hci_verify_block": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Block),
                              _i, _i, _i, _i, _p, _sz, _p]),
    "hci_verify_block_timed": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Block),
                                    _i, _i, _i, _i, _p, _sz, _p, _p]),
    "hci_verify_block_noalloc": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Block),
                                      _i, _i, _i, _i, _p]),
    "hci_accept": (_i, [_i, _i, _i, _i, _i, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "hci_slice_state": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Block),
                             _i, _i, _i, _i, _p, _p, _p]),
    "hci_verify_tree": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Tree), _i, _i, _i, _p, _sz,
                             _p]),
    "hci_accept_tree": (_i, [_i, _i, _i, _i, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "hci_slice_tree": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), ctypes.POINTER(Tree), _i, _i, _i, _p, _p,
                            _p]),
    "hci_prefill_workspace_bytes": (_sz, [ctypes.POINTER(Layer), _i, _i, _i]),
    "hci_prefill": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), _i, _i, _i, _p, _p, _p, _p, _p, _sz, _p]),
    "hci_linear_packed_elems": (_sz, [_i, _i]),
    "hci_linear_pack": (_i, [_i, _i, _p, _p, _p]),
    "hci_linear": (_i, [_i, _i, _i, _p, _p, _p, _p, _i, _p]),
    "hci_rmsnorm": (_i, [_i, _i, _p, _p, ctypes.c_float, _p, _p]),
    "hci_model_workspace_bytes": (_sz, [ctypes.POINTER(Model), _i, _i, _i, _i]),
    "hci_model_verify": (_i, [ctypes.POINTER(Model), ctypes.POINTER(ModelState), ctypes.POINTER(ModelBlock),
                              _i, _i, _i, _i, _p, _sz, _p]),
    "hci_model_slice": (_i, [ctypes.POINTER(Model), ctypes.POINTER(ModelState), ctypes.POINTER(ModelBlock),
                             _i, _i, _i, _i, _p, _p, _p]),
    "hci_draft_workspace_bytes": (_sz, [ctypes.POINTER(Drafter), _i, _i]),
    "hci_draft_logits": (_i, [ctypes.POINTER(Drafter), _i, _i, _p, _p, _p, _p, _sz, _p]),
    "hci_draft_sample": (_i, [_i, _i, _i, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p]),
    "hci_kv_cache_elems": (_sz, [ctypes.POINTER(Layer), _i, _i]),
    "hci_kv_write": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), _i, _i, _i, _i, _p, _p, _p]),
    "hci_kv_read": (_i, [ctypes.POINTER(Layer), ctypes.POINTER(State), _i, _i, _i, _i, _p, _p, _p]),
    "hci_probe_read": (_i, [_p, _sz, _p, _p]),
    "hci_probe_sink_words": (_i, []),
    "hci_probe_copy": (_i, [_p, _p, _sz, _p]),
}
for _name, (_res, _args) in EXPORTS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise HciError(rc, where)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def act_torch_dtype(act: int) -> torch.dtype:
    return torch.bfloat16 if act == BF16 else torch.float32


# ------------------------------------------------------------------ structs

def make_layer(d, taps_short, taps_outer, poles, heads, head_dim, act, w_short, w_outer, lam, beta, c) -> Layer:
    f32 = torch.float32
    return Layer(d, taps_short, taps_outer, poles, heads, head_dim, act,
                 _ptr(w_short, f32, "w_short"), _ptr(w_outer, f32, "w_outer"), _ptr(lam, f32, "lambda"),
                 _ptr(beta, f32, "beta"), _ptr(c, f32, "c"))


def make_state(act, kv_cap, short_win, outer_win, iir, k_cache, v_cache, kv_len, status=None) -> State:
    """status: optional [nb] int32 device tensor that receives the HCI_DS_* bits (uint32 words)."""
    at = act_torch_dtype(act)
    return State(kv_cap, _ptr(short_win, at, "short_win"), _ptr(outer_win, torch.float32, "outer_win"),
                 _ptr(iir, torch.float32, "iir"), _ptr(k_cache, at, "k_cache"), _ptr(v_cache, at, "v_cache"),
                 _ptr(kv_len, torch.int32, "kv_len"), _ptr(status, torch.int32, "status"))


def make_block(act, x, q, k, v, f, s, y, o) -> Block:
    at = act_torch_dtype(act)
    return Block(_ptr(x, at, "x"), _ptr(q, at, "q"), _ptr(k, at, "k"), _ptr(v, at, "v"),
                 _ptr(f, torch.float32, "f"), _ptr(s, torch.float32, "s"), _ptr(y, at, "y"), _ptr(o, at, "o"))


# ------------------------------------------------------------------ calls

def version() -> int:
    return _lib.hci_version()


def _text(fn, value) -> str:
    n = fn(value, None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    fn(value, buf, n + 1)
    return buf.value.decode()


def status_string(status: int) -> str:
    return _text(_lib.hci_status_string, status)


def device_status_string(bits: int) -> str:
    """Names of the HCI_DS_* bits set in a status word copied to the host."""
    return _text(_lib.hci_device_status_string, int(bits) & 0xFFFFFFFF)


def verify_workspace_bytes(layer: Layer, nb: int, nc: int, gamma: int, max_kv_len: int) -> int:
    return _lib.hci_verify_workspace_bytes(ctypes.byref(layer), nb, nc, gamma, max_kv_len)


def verify_block(layer: Layer, state: State, block: Block, nb: int, nc: int, gamma: int, max_kv_len: int,
                 ws: Optional[torch.Tensor], stream=None) -> None:
    wsp = _ptr(ws, None, "ws") if ws is not None else None
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.hci_verify_block(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(block), nb, nc, gamma,
                                 max_kv_len, wsp, nbytes, _stream(stream)), "hci_verify_block")


NOALLOC_SCRATCH_BYTES = 64 << 20


def verify_block_noalloc(layer: Layer, state: State, block: Block, nb: int, nc: int, gamma: int, max_kv_len: int,
                         stream=None) -> None:
    """hci_verify_block with the library's own scratch array as workspace (no allocation)."""
    _check(_lib.hci_verify_block_noalloc(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(block), nb, nc,
                                         gamma, max_kv_len, _stream(stream)), "hci_verify_block_noalloc")


def verify_block_timed(layer: Layer, state: State, block: Block, nb: int, nc: int, gamma: int, max_kv_len: int,
                       ws: Optional[torch.Tensor], events, stream=None) -> None:
    """events: a ctypes array of 4 hipEvent_t handles created by the caller (before the set-up
    kernel, before and after the streaming kernel, after the finish kernel)."""
    wsp = _ptr(ws, None, "ws") if ws is not None else None
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.hci_verify_block_timed(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(block), nb, nc, gamma,
                                       max_kv_len, wsp, nbytes, _stream(stream), ctypes.cast(events, _p)),
           "hci_verify_block_timed")


def accept(mode: int, nb: int, nc: int, gamma: int, vocab: int, temperature: float,
           target_logits, draft_logits, draft_tokens, uniforms,
           n_accepted, next_token, best_cand=None, margin=None, stream=None, status=None) -> None:
    """status: optional [nb] int32 device tensor receiving HCI_DS_* bits."""
    _check(_lib.hci_accept(mode, nb, nc, gamma, vocab, float(temperature),
                           _ptr(target_logits, torch.float32, "target_logits"),
                           _ptr(draft_logits, torch.float32, "draft_logits"),
                           _ptr(draft_tokens, torch.int32, "draft_tokens"),
                           _ptr(uniforms, torch.float64, "uniforms"),
                           _ptr(n_accepted, torch.int32, "n_accepted"), _ptr(next_token, torch.int32, "next_token"),
                           _ptr(best_cand, torch.int32, "best_cand"), _ptr(margin, torch.float64, "margin"),
                           _ptr(status, torch.int32, "status"), _stream(stream)), "hci_accept")


def slice_state(layer: Layer, state: State, block: Block, nb: int, nc: int, gamma: int, max_kv_len: int,
                n_accepted, best_cand=None, stream=None) -> None:
    _check(_lib.hci_slice_state(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(block), nb, nc, gamma,
                                max_kv_len, _ptr(n_accepted, torch.int32, "n_accepted"),
                                _ptr(best_cand, torch.int32, "best_cand"), _stream(stream)), "hci_slice_state")


def make_tree(act, parent, x, q, k, v, f, s, y, o) -> Tree:
    at = act_torch_dtype(act)
    return Tree(_ptr(parent, torch.int32, "parent"), _ptr(x, at, "x"), _ptr(q, at, "q"), _ptr(k, at, "k"),
                _ptr(v, at, "v"), _ptr(f, torch.float32, "f"), _ptr(s, torch.float32, "s"), _ptr(y, at, "y"),
                _ptr(o, at, "o"))


def verify_tree(layer: Layer, state: State, tree: Tree, nb: int, n: int, max_kv_len: int, ws, stream=None) -> None:
    _check(_lib.hci_verify_tree(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(tree), nb, n, max_kv_len,
                                _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "hci_verify_tree")


def accept_tree(mode: int, nb: int, n: int, vocab: int, temperature: float, parent, tokens, target_logits,
                draft_logits, uniforms, n_accepted, path, next_token, margin=None, status=None, stream=None) -> None:
    _check(_lib.hci_accept_tree(mode, nb, n, vocab, float(temperature), _ptr(parent, torch.int32, "parent"),
                                _ptr(tokens, torch.int32, "tokens"),
                                _ptr(target_logits, torch.float32, "target_logits"),
                                _ptr(draft_logits, torch.float32, "draft_logits"),
                                _ptr(uniforms, torch.float64, "uniforms"),
                                _ptr(n_accepted, torch.int32, "n_accepted"), _ptr(path, torch.int32, "path"),
                                _ptr(next_token, torch.int32, "next_token"), _ptr(margin, torch.float64, "margin"),
                                _ptr(status, torch.int32, "status"), _stream(stream)), "hci_accept_tree")


def slice_tree(layer: Layer, state: State, tree: Tree, nb: int, n: int, max_kv_len: int, n_accepted, path,
               stream=None) -> None:
    _check(_lib.hci_slice_tree(ctypes.byref(layer), ctypes.byref(state), ctypes.byref(tree), nb, n, max_kv_len,
                               _ptr(n_accepted, torch.int32, "n_accepted"), _ptr(path, torch.int32, "path"),
                               _stream(stream)), "hci_slice_tree")


def prefill_workspace_bytes(layer: Layer, nb: int, T: int, want_y: bool) -> int:
    return _lib.hci_prefill_workspace_bytes(ctypes.byref(layer), nb, T, 1 if want_y else 0)


def prefill(layer: Layer, state: State, nb: int, T: int, max_kv_len: int, x, k, v, y, ws, stream=None) -> None:
    _check(_lib.hci_prefill(ctypes.byref(layer), ctypes.byref(state), nb, T, max_kv_len,
                            _ptr(x, None, "x"), _ptr(k, None, "k"), _ptr(v, None, "v"), _ptr(y, None, "y"),
                            _ptr(ws, None, "ws"), ws.numel() * ws.element_size() if ws is not None else 0,
                            _stream(stream)), "hci_prefill")


def linear_packed_elems(K: int, N: int) -> int:
    return _lib.hci_linear_packed_elems(K, N)


def linear_pack(w, w_packed, stream=None) -> None:
    """w [K][N] bf16 -> w_packed (linear_packed_elems(K, N) bf16 elements)."""
    K, N = w.shape
    _check(_lib.hci_linear_pack(K, N, _ptr(w, torch.bfloat16, "w"), _ptr(w_packed, torch.bfloat16, "w_packed"),
                                _stream(stream)), "hci_linear_pack")


def linear(x, w_packed, N: int, y, residual=None, stream=None) -> None:
    """y [M][N] = x [M][K] w (+ residual); y bf16 or fp32."""
    M, K = x.shape
    _check(_lib.hci_linear(M, K, N, _ptr(x, torch.bfloat16, "x"), _ptr(w_packed, torch.bfloat16, "w_packed"),
                           _ptr(residual, torch.bfloat16, "residual"), _ptr(y, None, "y"),
                           1 if y.dtype == torch.float32 else 0, _stream(stream)), "hci_linear")


def rmsnorm(x, gamma, eps: float, y, stream=None) -> None:
    M, K = x.shape
    _check(_lib.hci_rmsnorm(M, K, _ptr(x, torch.bfloat16, "x"), _ptr(gamma, torch.float32, "gamma"), float(eps),
                            _ptr(y, torch.bfloat16, "y"), _stream(stream)), "hci_rmsnorm")


def model_workspace_bytes(model: Model, nb: int, nc: int, gamma: int, max_kv_len: int) -> int:
    return _lib.hci_model_workspace_bytes(ctypes.byref(model), nb, nc, gamma, max_kv_len)


def model_verify(model: Model, state: ModelState, block: ModelBlock, nb: int, nc: int, gamma: int, max_kv_len: int,
                 ws, stream=None) -> None:
    _check(_lib.hci_model_verify(ctypes.byref(model), ctypes.byref(state), ctypes.byref(block), nb, nc, gamma,
                                 max_kv_len, _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "hci_model_verify")


def model_slice(model: Model, state: ModelState, block: ModelBlock, nb: int, nc: int, gamma: int, max_kv_len: int,
                n_accepted, best_cand=None, stream=None) -> None:
    _check(_lib.hci_model_slice(ctypes.byref(model), ctypes.byref(state), ctypes.byref(block), nb, nc, gamma,
                                max_kv_len, _ptr(n_accepted, torch.int32, "n_accepted"),
                                _ptr(best_cand, torch.int32, "best_cand"), _stream(stream)), "hci_model_slice")


def draft_workspace_bytes(drafter: Drafter, nb: int, gamma: int) -> int:
    return _lib.hci_draft_workspace_bytes(ctypes.byref(drafter), nb, gamma)


def draft_logits(drafter: Drafter, nb: int, gamma: int, window, anchor, z, ws, stream=None) -> None:
    _check(_lib.hci_draft_logits(ctypes.byref(drafter), nb, gamma, _ptr(window, torch.bfloat16, "window"),
                                 _ptr(anchor, torch.int32, "anchor"), _ptr(z, torch.float32, "z"), _ptr(ws, None, "ws"),
                                 ws.numel() * ws.element_size(), _stream(stream)), "hci_draft_logits")


def draft_sample(nb: int, gamma: int, vocab: int, temperature: float, z, markov, anchor, uniforms, drafts,
                 draft_logits, margin=None, stream=None) -> None:
    _check(_lib.hci_draft_sample(nb, gamma, vocab, float(temperature), _ptr(z, torch.float32, "z"),
                                 _ptr(markov, torch.float32, "markov"), _ptr(anchor, torch.int32, "anchor"),
                                 _ptr(uniforms, torch.float64, "uniforms"), _ptr(drafts, torch.int32, "drafts"),
                                 _ptr(draft_logits, torch.float32, "draft_logits"),
                                 _ptr(margin, torch.float64, "margin"), _stream(stream)), "hci_draft_sample")


def kv_cache_elems(layer: Layer, nb: int, kv_cap: int) -> int:
    return _lib.hci_kv_cache_elems(ctypes.byref(layer), nb, kv_cap)


def kv_write(layer: Layer, state: State, nb: int, b: int, row0: int, k_rows, v_rows, stream=None) -> None:
    nrows = k_rows.shape[1]
    _check(_lib.hci_kv_write(ctypes.byref(layer), ctypes.byref(state), nb, b, row0, nrows,
                             _ptr(k_rows, None, "k_rows"), _ptr(v_rows, None, "v_rows"), _stream(stream)),
           "hci_kv_write")


def kv_read(layer: Layer, state: State, nb: int, b: int, row0: int, k_rows, v_rows, stream=None) -> None:
    nrows = k_rows.shape[1]
    _check(_lib.hci_kv_read(ctypes.byref(layer), ctypes.byref(state), nb, b, row0, nrows,
                            _ptr(k_rows, None, "k_rows"), _ptr(v_rows, None, "v_rows"), _stream(stream)),
           "hci_kv_read")


def probe_sink_words() -> int:
    return _lib.hci_probe_sink_words()


def probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    _check(_lib.hci_probe_read(_ptr(src, None, "src"), src.numel() * src.element_size(),
                               _ptr(sink, torch.float32, "sink"), _stream(stream)), "hci_probe_read")


def probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    _check(_lib.hci_probe_copy(_ptr(dst, None, "dst"), _ptr(src, None, "src"), src.numel() * src.element_size(),
                               _stream(stream)), "hci_probe_copy")
