"""The work list the device derives from kv_len, read back from the workspace and compared
with the Python transcription in tests/test_worklist.py (so the transcription cannot drift from
the device): the item count, the first-phase chunk c0, the phase count and the table of
(first item, items per head) per phase and sequence, for ragged batches of one to five
sequences, one and four candidate blocks, and empty prefixes.

Workspace header (bytes): the queue counter at 0, the item count at 4, c0 at 8, the phase
count at 12; from byte 256 the table [8 phases][nb] of int32 (base, n) pairs."""
import numpy as np
import pytest
import torch

from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import synth
from gpu_harness import Case, say
from test_worklist import KTILE, PHASE_MAX, _c0, _np, work_items

pytestmark = pytest.mark.gpu


def _expected_table(lens, heads, lim, resident, nq):
    tiles = [(min(max(L, 0), lim) + KTILE - 1) // KTILE for L in lens]
    c0 = _c0(sum(tiles) * heads, resident, nq)
    nph = _np(c0)
    table = np.zeros((PHASE_MAX, len(lens), 2), np.int64)
    base = 0
    for p in range(PHASE_MAX):
        for b, T in enumerate(tiles):
            n = 0
            if p < nph:
                c = c0 >> p
                s = T - (T >> p)
                e = T - (T >> (p + 1)) if p + 1 < nph else T
                n = (e - s + c - 1) // c
            table[p, b] = (base, n)
            base += heads * n
    return base, c0, nph, table


@pytest.mark.parametrize("lens,nc", [((8192,), 1), ((1000, 0, 33, 4096, 31), 1), ((16384, 32768, 51200, 65536), 4),
                                     ((0, 0), 1), ((262144,), 1)])
def test_device_work_list_matches_the_transcription(lens, nc):
    cfg = synth.scaled(synth.CONFIGS["mid8k"], d=256, heads=2, kv_lens=tuple(lens), nc=nc, gamma=12, mode="greedy")
    say(f"work list lens={lens} nc={nc}")
    case = Case(cfg, host_prefix=False)
    case.blk.ensure_workspace(cfg.max_kv_len).zero_()
    case.run_verify()
    torch.cuda.synchronize()
    ws = dv.to_host(case.blk.ws)
    hdr = ws[:16].view(np.int32)
    nb = len(lens)
    tab = ws[256:256 + PHASE_MAX * nb * 8].view(np.int32).reshape(PHASE_MAX, nb, 2)
    resident = torch.cuda.get_device_properties(0).multi_processor_count
    nq = nc * cfg.P
    total, c0, nph, table = _expected_table(lens, cfg.heads, cfg.max_kv_len, resident, nq)
    _, items = work_items(lens, cfg.heads, cfg.max_kv_len, resident, nq)
    assert total == len(items)
    assert (int(hdr[1]), int(hdr[2]), int(hdr[3])) == (total, c0, nph)
    np.testing.assert_array_equal(tab.astype(np.int64), table)
