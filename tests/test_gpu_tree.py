"""GPU token-tree verification, acceptance and slicing through the C ABI against
the fp64 oracle (oracle/tree.py, pinned against the chain oracle).

* verify: every node's f, s, y, o against the oracle on chains, stars, brooms
  and random trees of 1 to 64 nodes, fp32 and bf16 layers, ragged prefixes;
  and f, s, y bit for bit against the GPU chain verify over each root-to-leaf
  path (the tree kernel keeps the chain kernel's summation orders);
* accept: k, the accepted path, the next token bit-exact against the oracle
  (greedy and sampling, vocabularies 4 and 512; decisions away from rounding
  ties);
* a whole round (verify -> accept -> slice) equals sequential single-position
  steps along the accepted path: windows, IIR state, KV rows and lengths bit
  for bit;
* the 4 x 4-candidate workload (ragged 16384..65536-token prefixes) as
  prefix-sharing trees over a 4-letter vocabulary, at full size (attention
  checked on a sample of heads);
* guards: an invalid parent entry or a path that leaves the tree is reported
  (HCI_DS_TREE) and commits nothing.
Tolerances: tests/gpu_harness.py.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import tree as otree
from hybrid_conv_iir_amd import device as dv
from hybrid_conv_iir_amd import hci, synth
from gpu_harness import Case, assert_f32_close, assert_out_close, f64, say

pytestmark = pytest.mark.gpu

MARGIN = 1e-12


class TreeCase:
    """Layer, committed state (via the chain harness) and one tree per sequence on the device."""

    def __init__(self, cfg, parent, tokens, seed=0, host_prefix=True):
        self.parent = np.asarray(parent, np.int32)
        self.tokens = np.asarray(tokens, np.int32)
        self.n = self.parent.shape[1]
        kv_cap = (cfg.max_kv_len + max(self.n, cfg.P) + 31) // 32 * 32 + 32
        self.base = Case(cfg, seed=seed, host_prefix=host_prefix, kv_cap=kv_cap)
        self.cfg = cfg
        t = self.base.tables
        self.x, self.q, self.k, self.v = (t["E_x"][self.tokens], t["E_q"][self.tokens], t["E_k"][self.tokens],
                                          t["E_v"][self.tokens])
        self.tree = dv.DeviceTree(self.base.lay, cfg.nb, self.n, cfg.vocab)
        self.tree.set_inputs(self.parent, self.x, self.q, self.k, self.v)
        torch.cuda.synchronize()

    @property
    def st(self):
        return self.base.st

    def verify(self, max_kv_len=None):
        dv.verify_tree(self.base.lay, self.st, self.tree, self.cfg.max_kv_len if max_kv_len is None else max_kv_len)

    def oracle_verify(self, b, heads=None):
        st = self.base.oracle_state(b)
        q, k, v = self.q[b], self.k[b], self.v[b]
        if heads is not None:
            q, k, v = q[:, heads], k[:, heads], v[:, heads]
            st = oracle.SeqState(st.short_win, st.outer_win, st.iir, [blk[heads] for blk in st.k_blocks],
                                 [blk[heads] for blk in st.v_blocks])
        return otree.tree_verify(oracle.Layer.from_dict(self.base.params), st, self.parent[b], self.x[b], q, k, v)


def _check_verify(tc: TreeCase, heads=None):
    tc.verify()
    torch.cuda.synchronize()
    f, s, y, o = (dv.to_host(t) for t in (tc.tree.f, tc.tree.s, tc.tree.y, tc.tree.o))
    refs = []
    for b in range(tc.cfg.nb):
        ref = tc.oracle_verify(b, heads)
        refs.append(ref)
        tag = f"tree {tc.cfg.name} n={tc.n} b={b}"
        assert_f32_close(f[b], ref["f"], tag + " f")
        assert_f32_close(s[b], ref["s"], tag + " s")
        assert_out_close(tc.cfg, y[b], ref["y"], tag + " y")
        oo = o[b] if heads is None else o[b][:, heads]
        assert_out_close(tc.cfg, oo, ref["o"], tag + " o")
    assert [int(v) for v in dv.to_host(tc.st.status)] == [0] * tc.cfg.nb
    return refs


def _small_bf16(kv_lens):
    return synth.scaled(synth.CONFIGS["mid8k"], d=256, heads=2, kv_lens=kv_lens, vocab=64, mode="sample")


@pytest.mark.parametrize("kind", ["chain", "star", "broom", "random"])
@pytest.mark.parametrize("n", [1, 7, 33, 64])
def test_tree_verify_parity_fp32(kind, n):
    cfg = synth.scaled(synth.CONFIGS["tiny"], vocab=64)
    rng = np.random.default_rng(n * 7 + len(kind))
    parent = synth.random_tree(n, kind, rng)[None]
    tokens = rng.integers(0, cfg.vocab, (1, n))
    say(f"tree verify fp32 {kind} n={n}")
    _check_verify(TreeCase(cfg, parent, tokens))


@pytest.mark.parametrize("kind,n,lens", [("random", 40, (1000, 33)), ("broom", 64, (0, 4097)),
                                         ("star", 13, (31, 1)), ("chain", 13, (8192, 500))])
def test_tree_verify_parity_bf16(kind, n, lens):
    cfg = _small_bf16(lens)
    rng = np.random.default_rng(n + sum(lens))
    parent = np.stack([synth.random_tree(n, kind, rng) for _ in range(cfg.nb)])
    tokens = rng.integers(0, cfg.vocab, (cfg.nb, n))
    say(f"tree verify bf16 {kind} n={n} L={lens}")
    _check_verify(TreeCase(cfg, parent, tokens))


@pytest.mark.parametrize("act,shape", [("f32", "random"), ("bf16", "random"), ("f32", "trie"), ("bf16", "trie")])
def test_tree_conv_bits_equal_the_chain_over_each_path(act, shape):
    """f, s and y of every node carry the bits of the chain verify over its root-to-node path: a
    random 30-node tree (many root-to-leaf paths: the per-node FIR) and a trie of four candidate
    blocks sharing prefixes (few paths: the FIR along each path)."""
    cfg = synth.scaled(synth.CONFIGS["tiny"], vocab=64) if act == "f32" else _small_bf16((700,))
    rng = np.random.default_rng(21)
    if shape == "random":
        n = 30
        parent = synth.random_tree(n, "random", rng)[None]
    else:
        tr = synth.tree_round(synth.scaled(cfg, nc=4, gamma=12, vocab=4, kv_lens=cfg.kv_lens[:1]))
        parent = tr["parent"][:1]
        n = parent.shape[1]
    tokens = rng.integers(0, cfg.vocab, (1, n))
    tc = TreeCase(cfg, parent, tokens)
    say(f"tree vs chain bits ({act})")
    tc.verify()
    torch.cuda.synchronize()
    f, s, y, o = (dv.to_host(t)[0] for t in (tc.tree.f, tc.tree.s, tc.tree.y, tc.tree.o))
    leaves = [m for m in range(n) if m not in set(parent[0])]
    for m in leaves:
        path = otree.tree_path(parent[0], m)
        P = len(path)
        blk = dv.DeviceBlock(tc.base.lay, 1, 1, P - 1)
        blk.set_inputs(tc.x[:, path][:, None], tc.q[:, path][:, None], tc.k[:, path][:, None], tc.v[:, path][:, None])
        dv.verify(tc.base.lay, tc.st, blk, cfg.max_kv_len)
        torch.cuda.synchronize()
        cf, cs, cy, co = (dv.to_host(t)[0, 0] for t in (blk.f, blk.s, blk.y, blk.o))
        np.testing.assert_array_equal(f[path], cf, err_msg=f"f leaf {m}")
        np.testing.assert_array_equal(s[path], cs, err_msg=f"s leaf {m}")
        np.testing.assert_array_equal(y[path].view(np.uint8), cy.view(np.uint8), err_msg=f"y leaf {m}")
        assert_out_close(cfg, o[path], f64(co), f"o leaf {m}")


def _tree_round_case(cfg, n=None, seed=0, host_prefix=True):
    tr = synth.tree_round(cfg, n=n, seed=seed)
    tc = TreeCase(cfg, tr["parent"], tr["tokens"], seed=seed, host_prefix=host_prefix)
    tc.tree.set_accept_inputs(tr["tokens"], tr["target_logits"], tr["draft_logits"], tr["uniforms"])
    return tc, tr


def _oracle_accept(mode, tr, b, T):
    if mode == "greedy":
        return otree.tree_greedy_accept(tr["target_logits"][b], tr["parent"][b], tr["tokens"][b])
    return otree.tree_rejection_accept(tr["target_logits"][b], tr["draft_logits"][b], tr["parent"][b],
                                       tr["tokens"][b], tr["uniforms"][b], T)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("V,T,seed", [(4, 1.0, 0), (4, 0.5, 1), (512, 1.0, 2), (64, 2.0, 3)])
def test_tree_accept_parity(mode, V, T, seed):
    cfg = synth.scaled(synth.CONFIGS["tiny"], nc=4, vocab=V, temperature=T, kv_lens=(256, 256, 256))
    tc, tr = _tree_round_case(cfg, seed=seed)
    say(f"tree accept {mode} V={V} T={T} n={tr['n']}")
    dv.accept_tree(tc.tree, hci.GREEDY if mode == "greedy" else hci.SAMPLE, T, status=tc.st.status)
    torch.cuda.synchronize()
    n_acc, path, nxt = (dv.to_host(t) for t in (tc.tree.n_acc, tc.tree.path, tc.tree.next))
    for b in range(cfg.nb):
        k, rpath, rnext, marg = _oracle_accept(mode, tr, b, T)
        assert marg > MARGIN, f"near-tie decision in the oracle: {marg}"
        assert int(n_acc[b]) == k and int(nxt[b]) == rnext, (b, int(n_acc[b]), k, int(nxt[b]), rnext)
        assert list(path[b, : k + 1]) == rpath and (path[b, k + 1:] == -1).all()
    assert [int(v) for v in dv.to_host(tc.st.status)] == [0] * cfg.nb


def _clone_state(src):
    st = dv.DeviceState(src.layer, src.nb, src.kv_cap)
    for a in ("short_win", "outer_win", "iir", "k_cache", "v_cache", "kv_len"):
        getattr(st, a).copy_(getattr(src, a))
    return st


@pytest.mark.parametrize("cfgname,mode", [("tiny", "sample"), ("mid8k", "greedy"), ("mid8k", "sample")])
def test_tree_round_equals_sequential_steps(cfgname, mode):
    """verify_tree + accept_tree + slice_tree = sequential single-position steps along the accepted
    path (windows, IIR state, KV rows, lengths: bit for bit)."""
    base = synth.CONFIGS[cfgname]
    cfg = synth.scaled(base, nc=4, vocab=4, mode=mode, kv_lens=(base.kv_lens[0], base.kv_lens[0] // 2 + 3))
    tc, tr = _tree_round_case(cfg, seed=5, host_prefix=False)
    before = _clone_state(tc.st)
    say(f"tree round {cfgname} {mode} n={tr['n']}")
    tc.verify()
    dv.accept_tree(tc.tree, hci.GREEDY if mode == "greedy" else hci.SAMPLE, cfg.temperature, status=tc.st.status)
    dv.slice_tree(tc.base.lay, tc.st, tc.tree, cfg.max_kv_len)
    torch.cuda.synchronize()
    n_acc, path = dv.to_host(tc.tree.n_acc), dv.to_host(tc.tree.path)
    blk1 = dv.DeviceBlock(tc.base.lay, cfg.nb, 1, 0)
    acc1 = dv.DeviceAccept(cfg.nb, 1, 0, cfg.vocab)
    steps = int(n_acc.max()) + 1
    for i in range(steps):
        # one position per sequence; a sequence whose path is shorter repeats no step: its extra
        # steps are run on a scratch copy and discarded below
        rows = [int(path[b, min(i, int(n_acc[b]))]) for b in range(cfg.nb)]
        blk1.set_inputs(tc.x[np.arange(cfg.nb), rows][:, None, None], tc.q[np.arange(cfg.nb), rows][:, None, None],
                        tc.k[np.arange(cfg.nb), rows][:, None, None], tc.v[np.arange(cfg.nb), rows][:, None, None])
        lens_now = dv.to_host(before.kv_len).copy()
        dv.verify(tc.base.lay, before, blk1, int(lens_now.max()))
        acc1.n_acc.zero_()
        keep = torch.tensor([i <= int(n_acc[b]) for b in range(cfg.nb)], device="cuda")
        saved = {a: getattr(before, a).clone() for a in ("short_win", "outer_win", "iir", "kv_len")}
        dv.slice_state(tc.base.lay, before, blk1, acc1, int(lens_now.max()))
        for a, t in saved.items():                      # sequences already done keep their state
            cur = getattr(before, a)
            cur.copy_(torch.where(keep.view(-1, *([1] * (cur.dim() - 1))), cur, t))
    torch.cuda.synchronize()
    a, b_ = tc.st.snapshot(), before.snapshot()
    for key in a:
        np.testing.assert_array_equal(a[key], b_[key], err_msg=key)
    for b in range(cfg.nb):
        L0, k = cfg.kv_lens[b], int(n_acc[b])
        kr, vr = tc.st.read_rows(b, L0, k + 1)
        ks, vs = before.read_rows(b, L0, k + 1)
        assert torch.equal(kr, ks) and torch.equal(vr, vs), f"KV rows b={b}"
    assert [int(v) for v in dv.to_host(tc.st.status)] == [0] * cfg.nb


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_multi4x4_as_trees_full_size(mode):
    """The 4 x 4-candidate workload (ragged 16384..65536-token prefixes, gamma 12) with drafts over a
    4-letter vocabulary, so candidates share prefixes; every node against the oracle (attention on 4
    of 32 heads), acceptance bit-exact, slice against the oracle."""
    cfg = synth.scaled(synth.CONFIGS["multi4x4"], vocab=4, mode=mode)
    tc, tr = _tree_round_case(cfg, seed=1)
    heads = [0, 11, 22, 31]
    say(f"multi4x4 trees {mode}: n={tr['n']} tries={tr['trie_sizes']}")
    refs = _check_verify(tc, heads)
    dv.accept_tree(tc.tree, hci.GREEDY if mode == "greedy" else hci.SAMPLE, cfg.temperature, status=tc.st.status)
    dv.slice_tree(tc.base.lay, tc.st, tc.tree, cfg.max_kv_len)
    torch.cuda.synchronize()
    n_acc, path, nxt = (dv.to_host(t) for t in (tc.tree.n_acc, tc.tree.path, tc.tree.next))
    snap = tc.st.snapshot()
    for b in range(cfg.nb):
        k, rpath, rnext, marg = _oracle_accept(mode, tr, b, cfg.temperature)
        assert marg > MARGIN
        assert int(n_acc[b]) == k and list(path[b, : k + 1]) == rpath and int(nxt[b]) == rnext
        new = otree.tree_slice(tc.base.oracle_state(b), tc.x[b], refs[b], tc.k[b], tc.v[b], rpath)
        np.testing.assert_array_equal(f64(snap["short_win"][b]), new.short_win)
        assert_f32_close(snap["outer_win"][b], new.outer_win, f"b={b} outer_win")
        assert_f32_close(snap["iir"][b], new.iir, f"b={b} iir")
        assert int(snap["kv_len"][b]) == cfg.kv_lens[b] + k + 1
        kr, _ = tc.st.read_rows(b, cfg.kv_lens[b], k + 1)
        np.testing.assert_array_equal(dv.to_host(kr), np.asarray(tc.k[b][rpath]).transpose(1, 0, 2))


def test_invalid_tree_and_path_commit_nothing():
    cfg = synth.scaled(synth.CONFIGS["tiny"], nc=3, vocab=8, kv_lens=(256, 256))
    tc, tr = _tree_round_case(cfg, seed=2)
    parent = tr["parent"].copy()
    parent[1, 3] = 5                                   # sequence 1: a parent after its child
    tc.tree.parent.copy_(torch.from_numpy(parent))
    before = tc.st.snapshot()
    say("tree guards: invalid parent entry")
    tc.verify()
    dv.accept_tree(tc.tree, hci.SAMPLE, 1.0, status=tc.st.status)
    dv.slice_tree(tc.base.lay, tc.st, tc.tree, cfg.max_kv_len)
    torch.cuda.synchronize()
    st = [int(v) for v in dv.to_host(tc.st.status)]
    assert st[0] == 0 and st[1] & hci.DS_TREE, [hci.device_status_string(v) for v in st]
    assert int(dv.to_host(tc.tree.n_acc)[1]) == -1
    after = tc.st.snapshot()
    for key in before:
        np.testing.assert_array_equal(after[key][1], before[key][1], err_msg=key)
    assert int(after["kv_len"][0]) > int(before["kv_len"][0])
    # a path that skips a level of the tree is refused by slicing
    tc2, tr2 = _tree_round_case(synth.scaled(cfg, kv_lens=(256,)), seed=3)
    par = tr2["parent"][0]
    deep = max(range(tc2.n), key=lambda m: len(otree.tree_path(par, m)))
    p = otree.tree_path(par, deep)
    assert len(p) >= 3
    bad_path = np.full((1, tc2.n), -1, np.int32)
    bad_path[0, : len(p) - 1] = [p[0]] + p[2:]
    tc2.tree.path.copy_(torch.from_numpy(bad_path))
    tc2.tree.n_acc.fill_(len(p) - 2)
    before2 = tc2.st.snapshot()
    say("tree guards: a path that leaves the tree")
    dv.slice_tree(tc2.base.lay, tc2.st, tc2.tree, 256)
    torch.cuda.synchronize()
    assert [int(v) for v in dv.to_host(tc2.st.status)] == [hci.DS_TREE]
    after2 = tc2.st.snapshot()
    for key in before2:
        np.testing.assert_array_equal(after2[key], before2[key], err_msg=key)
