"""The split of the KV prefixes into work items (CPU).

The prefix-streaming kernels take items from a queue and write one partial
per item; the workspace holds a partial slot for every item the host's bound
allows.  This test transcribes the device's work list (phase p covers the
next half of every prefix in chunks of c0 >> p tiles, c0 = max(32,
ceil(W / sR)) with s = 2, or 1 above 32 queries per sequence, at most 8
phases) and checks, over many ragged batches, that
the items tile every (sequence, head) prefix exactly once and that their
count never exceeds what hci_verify_workspace_bytes provides.
"""
import ctypes
import random

import numpy as np
import pytest

KTILE, CHUNK_MIN, PHASE_MAX = 32, 32, 8


def _c0(total_tiles, resident, nq):
    half = (1 if nq > 32 else 2) * max(resident, 1)
    return min(max((total_tiles + half - 1) // half, CHUNK_MIN), 1 << 28)


def _np(c0):
    n = 1
    while n < PHASE_MAX and (c0 >> n) >= CHUNK_MIN:
        n += 1
    return n


def work_items(lens, heads, lim, resident, nq=13):
    tiles = [(min(max(L, 0), lim) + KTILE - 1) // KTILE for L in lens]
    c0 = _c0(sum(tiles) * heads, resident, nq)
    nph = _np(c0)
    items = []
    for p in range(nph):
        c = c0 >> p
        for b, T in enumerate(tiles):
            s = T - (T >> p)
            e = T - (T >> (p + 1)) if p + 1 < nph else T
            n = (e - s + c - 1) // c
            for h in range(heads):
                for j in range(n):
                    t0 = s + j * c
                    items.append((b, h, t0, min(t0 + c, e)))
    return tiles, items


def _workspace_items(lib, layer, nb, nc, gamma, max_len):
    """Partial slots in the workspace the host plans for (after the header: 256 bytes for the
    queue counter, then the work-list table of 8 phases x nb (base, count) int32 pairs, rounded
    up to 256 bytes)."""
    nbytes = lib.hci_verify_workspace_bytes(ctypes.byref(layer), nb, nc, gamma, max_len)
    nq = nc * (gamma + 1)
    per_item = nq * layer.head_dim * 4 + nq * 2 * 4
    header = 256 + (8 * nb * 2 * 4 + 255) // 256 * 256
    return (nbytes - header) // per_item


@pytest.fixture(scope="module")
def hci():
    from hybrid_conv_iir_amd import hci as h
    return h


def _layer(hci, heads, head_dim=128):
    p = ctypes.c_void_p(16)
    return hci.Layer(d=heads * head_dim, taps_short=3, taps_outer=128, poles=16, heads=heads, head_dim=head_dim,
                     act_dtype=hci.BF16, w_short=p, w_outer=p, lambda_=p, beta=p, c=p)


@pytest.mark.parametrize("name,lens,heads,nq", [("long-context", [262144], 32, 13), ("wide", [131072], 64, 13),
                                                ("4 ragged", [16384, 32768, 51200, 65536], 32, 52),
                                                ("mid", [8192], 32, 13)])
def test_workloads_tile_their_prefixes(hci, name, lens, heads, nq):
    tiles, items = work_items(lens, heads, max(lens), 256, nq)
    cover = {}
    for b, h, t0, t1 in items:
        assert t1 > t0
        cover.setdefault((b, h), []).append((t0, t1))
    for b, T in enumerate(tiles):
        for h in range(heads):
            spans = sorted(cover[(b, h)])
            assert spans[0][0] == 0 and spans[-1][1] == T
            assert all(a[1] == c[0] for a, c in zip(spans, spans[1:]))      # contiguous, no overlap


def test_item_count_never_exceeds_the_workspace(hci):
    lib = hci._lib
    rng = random.Random(7)
    checked = 0
    for _ in range(400):
        nb = rng.choice([1, 1, 2, 3, 4, 7])
        heads = rng.choice([1, 8, 32, 64])
        nc, gamma = rng.choice([(1, 12), (1, 6), (4, 12), (2, 0)])
        max_len = rng.choice([1, 31, 33, 1000, 8192, 65536, 262144, rng.randint(1, 300000)])
        lens = [rng.choice([max_len, rng.randint(0, max_len), 0]) for _ in range(nb)]
        if heads * nb * (max_len // KTILE) > 2_000_000:
            continue
        layer = _layer(hci, heads)
        cap = _workspace_items(lib, layer, nb, nc, gamma, max_len)
        # the device plans for its own CU count; without a GPU the host assumes 256 CUs, one
        # streaming workgroup each
        _, items = work_items(lens, heads, max_len, 256, nc * (gamma + 1))
        assert len(items) <= cap, (nb, heads, nc, gamma, max_len, lens, len(items), cap)
        checked += 1
    assert checked > 300


def test_empty_prefixes_have_no_items():
    _, items = work_items([0, 0], 8, 1000, 256)
    assert items == []
