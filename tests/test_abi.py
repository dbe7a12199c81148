"""The C-ABI library loads and exports every symbol include/hci.h declares;
host-side argument checks reject bad calls before any launch (CPU only: no
call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hci.h")
LIB = os.path.join(ROOT, "hybrid_conv_iir_amd", "libhci.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hci_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libhci.so is not built: run `python -m hybrid_conv_iir_amd.build`")
    return ctypes.CDLL(LIB)


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("hci_verify_block", "hci_accept", "hci_slice_state"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_symbol():
    from hybrid_conv_iir_amd import hci
    assert sorted(hci.EXPORTS) == _declared()


def test_status_strings(lib):
    from hybrid_conv_iir_amd import hci
    assert hci.version() == 200
    for code in (0, -1, -2, -3, -4, -5):
        assert hci.status_string(code).startswith("HCI")
    f = hci._lib.hci_status_string
    full = hci.status_string(hci.EINVAL)
    assert f(hci.EINVAL, None, 0) == len(full)                 # sizing call
    buf = ctypes.create_string_buffer(b"\xff" * 8)
    assert f(hci.EINVAL, buf, 5) == len(full)                  # truncated, NUL-terminated
    assert buf.raw[:5] == full[:4].encode() + b"\0" and buf.raw[5:8] == b"\xff" * 3
    assert f(hci.EINVAL, None, 5) == hci.EINVAL


def test_device_status_strings():
    from hybrid_conv_iir_amd import hci
    assert hci.device_status_string(0) == "none"
    assert hci.device_status_string(hci.DS_NONFINITE | hci.DS_KV_LEN) == "HCI_DS_NONFINITE|HCI_DS_KV_LEN"
    assert hci.device_status_string(hci.DS_K_RANGE) == "HCI_DS_K_RANGE"
    assert hci.device_status_string(hci.DS_CAND_RANGE | hci.DS_DRAFT_ID) == "HCI_DS_CAND_RANGE|HCI_DS_DRAFT_ID"
    assert hci.device_status_string(0x100) == "unknown 0x100"
    assert hci._lib.hci_device_status_string(1, None, 3) == hci.EINVAL


def _layer(hci, **kw):
    p = dict(d=64, taps_short=3, taps_outer=7, poles=16, heads=1, head_dim=64, act_dtype=hci.F32,
             w_short=8, w_outer=8, lambda_=8, beta=8, c=8)
    p.update(kw)
    return hci.Layer(**p)


def test_host_validation_rejects_before_launch():
    from hybrid_conv_iir_amd import hci
    lib = hci._lib
    lay = _layer(hci)
    st = hci.State(kv_cap=512, short_win=16, outer_win=16, iir=16, k_cache=16, v_cache=16, kv_len=16)
    blk = hci.Block(x=16, q=16, k=16, v=16, f=16, s=16, y=16, o=16)
    V = ctypes.byref
    # null layer / bad dims / bad dtype
    assert lib.hci_verify_block(None, V(st), V(blk), 1, 1, 6, 256, None, 0, None) == hci.EINVAL
    assert lib.hci_verify_block(V(_layer(hci, d=0)), V(st), V(blk), 1, 1, 6, 256, None, 0, None) == hci.EINVAL
    assert lib.hci_verify_block(V(_layer(hci, act_dtype=7)), V(st), V(blk), 1, 1, 6, 256, None, 0, None) == hci.EINVAL
    assert lib.hci_verify_block(V(_layer(hci, act_dtype=hci.BF16, head_dim=96)), V(st), V(blk), 1, 1, 6, 256,
                                None, 0, None) == hci.EUNSUPPORTED
    assert lib.hci_verify_block(V(lay), V(st), V(blk), 1, 1, -1, 256, None, 0, None) == hci.EINVAL
    assert lib.hci_verify_block(V(lay), V(st), V(blk), 1, 1, 64, 256, None, 0, None) == hci.EUNSUPPORTED
    assert lib.hci_verify_block(V(lay), V(st), V(blk), 1, 16, 6, 256, None, 0, None) == hci.EUNSUPPORTED
    # capacity: 506 + 6 + 1 > 512
    assert lib.hci_verify_block(V(lay), V(st), V(blk), 1, 1, 6, 506, None, 0, None) == hci.ECAPACITY
    bad_cap = hci.State(kv_cap=500, short_win=16, outer_win=16, iir=16, k_cache=16, v_cache=16, kv_len=16)
    assert lib.hci_verify_block(V(lay), V(bad_cap), V(blk), 1, 1, 6, 256, None, 0, None) == hci.EINVAL
    # missing block pointer, misaligned q
    assert lib.hci_verify_block(V(lay), V(st), V(hci.Block(x=16, q=16, k=16, v=16, f=16, s=16, y=16, o=None)),
                                1, 1, 6, 256, None, 0, None) == hci.EINVAL
    assert lib.hci_verify_block(V(lay), V(st), V(hci.Block(x=16, q=18, k=16, v=16, f=16, s=16, y=16, o=16)),
                                1, 1, 6, 256, None, 0, None) == hci.EINVAL
    # workspace missing when the prefix is non-empty
    assert lib.hci_verify_block(V(lay), V(st), V(blk), 1, 1, 6, 256, None, 0, None) == hci.EWORKSPACE


def test_accept_and_slice_validation():
    from hybrid_conv_iir_amd import hci
    lib = hci._lib
    p = 4096
    assert lib.hci_accept(3, 1, 1, 6, 512, 1.0, p, p, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(-1, 1, 1, 6, 512, 1.0, p, p, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.SAMPLE_RECURSIVE, 1, 2, 6, 512, -1.0, p, p, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.SAMPLE_RECURSIVE, 1, 2, 6, 512, 1.0, p, p, p, None, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.SAMPLE_RECURSIVE, 1, 65, 6, 512, 1.0, p, p, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.SAMPLE, 1, 1, 6, 512, 0.0, p, p, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.SAMPLE, 1, 1, 6, 512, 1.0, p, None, p, p, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.GREEDY, 1, 1, 6, 0, 1.0, p, None, p, None, p, p, p, p, None, None) == hci.EINVAL
    assert lib.hci_accept(hci.GREEDY, 1, 1, 6, 1 << 20, 1.0, p, None, p, None, p, p, p, p, None, None) == hci.EUNSUPPORTED
    assert lib.hci_accept(hci.GREEDY, 1, 1, 6, 512, 1.0, None, None, p, None, p, p, p, p, None, None) == hci.EINVAL
    lay = _layer(hci)
    st = hci.State(kv_cap=512, short_win=16, outer_win=16, iir=16, k_cache=16, v_cache=16, kv_len=16)
    blk = hci.Block(x=16, q=16, k=16, v=16, f=16, s=16, y=16, o=16)
    V = ctypes.byref
    assert lib.hci_slice_state(V(lay), V(st), V(blk), 1, 1, 6, 256, None, None, None) == hci.EINVAL
    assert lib.hci_slice_state(V(lay), V(st), V(blk), 1, 2, 6, 256, p, None, None) == hci.EINVAL
    assert lib.hci_slice_state(V(lay), V(st), V(blk), 1, 1, 6, 510, p, None, None) == hci.ECAPACITY
    assert lib.hci_kv_write(V(lay), V(st), 1, 1, 0, 4, p, p, None) == hci.EINVAL        # b >= nb
    assert lib.hci_kv_write(V(lay), V(st), 1, 0, 500, 40, p, p, None) == hci.ECAPACITY
    assert lib.hci_kv_read(V(lay), V(st), 1, 0, 0, 4, None, p, None) == hci.EINVAL
    assert lib.hci_kv_cache_elems(V(lay), 2, 512) == 2 * 1 * 512 * 64
    assert lib.hci_probe_read(p + 1, 1024, p, None) == hci.EINVAL
    assert lib.hci_probe_copy(p, p, 1000, None) == hci.EINVAL


def test_kv_tile_layout_is_a_permutation():
    """Host-side mirror check of the documented tile layout: every (row, dim) of a
    32-key tile maps to a distinct slot (so kv_write/kv_read round-trip)."""
    from hybrid_conv_iir_amd import hci
    assert hci.KV_TILE == 32
    # re-derive the documented formulas independently and check bijectivity
    for Dh in (64, 128):
        ks, vs = set(), set()
        for w in range(32):
            for dd in range(Dh):
                u, m, j, g, e = w >> 4, w & 15, dd >> 5, (dd >> 3) & 3, dd & 7
                ks.add(((((u * (Dh >> 5) + j) * 4 + g) * 16 + m) * 8 + e))
                half, r = w >> 4, w & 15
                vs.add((((dd >> 4) * 4 + (r >> 2)) * 16 + (dd & 15)) * 8 + (r & 3) + 4 * half)
        assert ks == set(range(32 * Dh)) and vs == set(range(32 * Dh))
