"""Pins of the oracle's tree (trie / star) verify functions, CPU only.

DSSD fast.py, _set_rows, _star_cycle and _tree_cycle: the rows of a sequence are
the nodes of a draft tree in creation order. Node i sits at position pos + depth(i),
writes its K/V at slot pos + i and attends to slots 0..pos plus the slots of its
own path. Verification walks the tree from the root, and the accepted path's K/V
moves to contiguous slots. Each pin below checks the tree functions against
something other than themselves:
  * the chain functions (a chain is a tree whose parent list is i - 1);
  * PyTorch's CPU attention on keys gathered by hand;
  * one-row decoding on a pool where the path was written contiguously;
  * a brute-force acceptance rule stated over all nodes at once;
  * the lossless invariant on the toy model.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.toy_lm import ToyLM
from tests import pool_layout as PL
from tests.test_oracle_pins import _small_inputs


def _random_parents(rng, k, chain_bias=0.5):
    """parent list [k + 1] in creation order: parent[0] = -1, parent[i] in [0, i)."""
    par = [-1]
    for i in range(1, k + 1):
        par.append(i - 1 if rng.uniform() < chain_bias else int(rng.integers(0, i)))
    return np.array(par, np.int32)


def _depths(par):
    d = [0] * len(par)
    for i in range(1, len(par)):
        d[i] = d[par[i]] + 1
    return d


def _path(par, j):
    p = []
    while j != 0:
        p.append(j)
        j = par[j]
    return p[::-1]


def _tree_inputs(seed, B=3, k=(0, 7), chain_bias=0.5, **kw):
    x = _small_inputs(seed, B=B, k=k, **kw)
    rng = np.random.default_rng(seed + 1000)
    kmax = int(x["k"].max())
    parent = np.full((B, kmax + 1), 0, np.int32)
    for s in range(B):
        parent[s, :x["k"][s] + 1] = _random_parents(rng, int(x["k"][s]), chain_bias)
    return x, parent, kmax


def _run_tree(x, parent, kmax, k_pool=None, v_pool=None):
    off, st = oracle.validate(x["pt"], x["max_pages"], x["n_pages"], x["pos"], x["k"], 64, x["B"], x["R"])
    oracle.validate_tree(parent, kmax, x["k"], x["B"], st)
    kp = (x["k_pool"] if k_pool is None else k_pool).copy()
    vp = (x["v_pool"] if v_pool is None else v_pool).copy()
    oracle.append_kv(x["k_new"], x["v_new"], kp, vp, x["pt"], x["max_pages"], x["pos"], x["k"], off, st,
                     x["B"], x["Hkv"], x["D"])
    out = oracle.verify_attn_tree(x["q"], kp, vp, x["pt"], x["max_pages"], x["pos"], x["k"], parent, kmax, off,
                                  st, x["B"], x["R"], x["Hq"], x["Hkv"], x["D"], 1 / math.sqrt(x["D"]))
    return out, kp, vp, off, st


def test_validate_tree_flags():
    k = np.array([3, 3, 3, 0, 2], np.int32)
    parent = np.array([[-1, 0, 1, 1],      # fine
                       [-1, 0, 2, 0],      # parent not before the child
                       [0, 0, 1, 2],       # root must have parent -1
                       [-1, 7, 7, 7],      # k = 0: only the root is read
                       [-1, -1, 0, 9]],    # a node without a parent (entries past k unread)
                      np.int32)
    st = np.zeros(5, np.int32)
    oracle.validate_tree(parent, 3, k, 5, st)
    assert list(st) == [0, oracle.BAD_TREE, oracle.BAD_TREE, 0, oracle.BAD_TREE]


def test_chain_tree_equals_chain_attention_exactly():
    x = _small_inputs(11, B=4, k=(0, 6))
    kmax = int(x["k"].max())
    parent = np.tile(np.arange(-1, kmax, dtype=np.int32), (x["B"], 1))
    out_t, kp_t, vp_t, _, st = _run_tree(x, parent, kmax)
    assert (st == 0).all()
    off, st2 = oracle.validate(x["pt"], x["max_pages"], x["n_pages"], x["pos"], x["k"], 64, x["B"], x["R"])
    kp, vp = x["k_pool"].copy(), x["v_pool"].copy()
    oracle.append_kv(x["k_new"], x["v_new"], kp, vp, x["pt"], x["max_pages"], x["pos"], x["k"], off, st2,
                     x["B"], x["Hkv"], x["D"])
    out_c = oracle.verify_attn(x["q"], kp, vp, x["pt"], x["max_pages"], x["pos"], x["k"], off, st2, x["B"],
                               x["R"], x["Hq"], x["Hkv"], x["D"], 1 / math.sqrt(x["D"]))
    np.testing.assert_array_equal(out_t, out_c)


def _gather_slots(x, kp, vp, s, slots):
    """K/V of sequence s at the given slots as float64 [Hkv, n, D], indexed independently."""
    idx = np.asarray(slots)
    pages = x["pt"][s, idx // 16]
    Kl, Vl = PL.unpack(kp, PL.k_offsets(x["D"])), PL.unpack(vp, PL.v_offsets(x["D"]))
    K = oracle.bf16_bits_to_f64(Kl[pages, :, idx % 16, :])
    V = oracle.bf16_bits_to_f64(Vl[pages, :, idx % 16, :])
    return np.transpose(K, (1, 0, 2)), np.transpose(V, (1, 0, 2))


@pytest.mark.parametrize("seed,chain_bias", [(12, 0.5), (13, 0.0), (14, 0.9)])
def test_tree_attention_matches_torch_sdpa_on_path_keys(seed, chain_bias):
    """Library routine: PyTorch CPU scaled_dot_product_attention (fp64, GQA) over the
    committed slots 0..pos and the slots of the row's own path."""
    x, parent, kmax = _tree_inputs(seed, B=4, k=(2, 9), chain_bias=chain_bias, Hq=8, Hkv=2, D=32)
    out, kp, vp, off, st = _run_tree(x, parent, kmax)
    assert (st == 0).all()
    for s in range(x["B"]):
        P = int(x["pos"][s])
        for j in range(x["k"][s] + 1):
            slots = list(range(P + 1)) + [P + u for u in _path(parent[s], j)]
            K, V = _gather_slots(x, kp, vp, s, slots)
            qq = torch.from_numpy(oracle.bf16_bits_to_f64(x["q"][off[s] + j]))
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq[:, None, :], torch.from_numpy(K), torch.from_numpy(V), scale=1 / math.sqrt(x["D"]),
                enable_gqa=True)[:, 0, :]
            np.testing.assert_allclose(out[off[s] + j], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_tree_rows_equal_one_row_decode_after_compaction():
    """Node j's row equals a one-row call at position pos + depth(j) on a pool where
    the K/V of its path was appended contiguously at pos + 1.. (the compacted layout
    the next cycle sees), exactly: same keys, same order."""
    x, parent, kmax = _tree_inputs(15, B=3, k=(3, 8), chain_bias=0.3)
    out, kp_tree, _, off, st = _run_tree(x, parent, kmax)
    assert (st == 0).all()
    for s in range(x["B"]):
        dep = _depths(parent[s])
        for j in range(x["k"][s] + 1):
            kp1, vp1 = x["k_pool"].copy(), x["v_pool"].copy()
            chain = [0] + _path(parent[s], j)           # root then the path, one row per depth
            for d, u in enumerate(chain):
                r = off[s] + u
                y = dict(x, B=1, R=1, pos=x["pos"][s:s + 1] + d, k=np.zeros(1, np.int32),
                         pt=x["pt"][s:s + 1], k_new=x["k_new"][r:r + 1], v_new=x["v_new"][r:r + 1])
                o_, st1 = oracle.validate(y["pt"], y["max_pages"], y["n_pages"], y["pos"], y["k"], 64, 1, 1)
                oracle.append_kv(y["k_new"], y["v_new"], kp1, vp1, y["pt"], y["max_pages"], y["pos"], y["k"],
                                 o_, st1, 1, x["Hkv"], x["D"])
            pj = np.array([x["pos"][s] + dep[j]], np.int32)
            o_, st1 = oracle.validate(x["pt"][s:s + 1], x["max_pages"], x["n_pages"], pj, np.zeros(1, np.int32),
                                      64, 1, 1)
            o1 = oracle.verify_attn(x["q"][off[s] + j:off[s] + j + 1], kp1, vp1, x["pt"][s:s + 1],
                                    x["max_pages"], pj, np.zeros(1, np.int32), o_, st1, 1, 1, x["Hq"], x["Hkv"],
                                    x["D"], 1 / math.sqrt(x["D"]))
            np.testing.assert_array_equal(o1[0], out[off[s] + j])


def test_star_children_see_root_not_siblings():
    """Star (depth-1 tree, fast.py _star_cycle): a child's output does not change when
    a sibling's K/V changes, and does when the root's K/V changes."""
    x = _small_inputs(16, B=1, k=(5, 5))
    parent = np.array([[-1, 0, 0, 0, 0, 0]], np.int32)
    out, *_ = _run_tree(x, parent, 5)
    rng = np.random.default_rng(3)
    kn = x["k_new"].copy()
    kn[3] = oracle.f32_to_bf16_bits(rng.standard_normal(kn[3].shape).astype(np.float32))
    out2, *_ = _run_tree(dict(x, k_new=kn), parent, 5)
    for j in (0, 1, 2, 4, 5):
        np.testing.assert_array_equal(out2[j], out[j])
    assert not np.array_equal(out2[3], out[3])
    kn = x["k_new"].copy()
    kn[0] = oracle.f32_to_bf16_bits(rng.standard_normal(kn[0].shape).astype(np.float32))
    out3, *_ = _run_tree(dict(x, k_new=kn), parent, 5)
    for j in range(6):
        assert not np.array_equal(out3[j], out[j])


def test_bad_tree_rows_untouched():
    x, parent, kmax = _tree_inputs(17, B=3, k=(3, 5))
    parent[1, 2] = 2
    out, kp, vp, off, st = _run_tree(x, parent, kmax)
    assert st[1] == oracle.BAD_TREE and st[0] == 0 and st[2] == 0
    assert np.isnan(out[off[1]:off[1] + x["k"][1] + 1]).all()
    assert not np.isnan(out[off[0]:off[0] + x["k"][0] + 1]).any()


# --------------------------------------------------------------------------- acceptance
def _accept1(g, toks, par, d2t=None, nd=0, V=50, pos=10):
    k = len(toks)
    return oracle.tree_accept(np.array(g, np.int32), np.array([toks], np.int32), k, np.array([k], np.int32),
                              np.array([par], np.int32), d2t, nd, V, 1, k + 1, np.array([pos], np.int32))


@pytest.mark.parametrize("g,toks,par,acc,path,emit", [
    # star: the root's target picks the child; the child's target is the bonus
    ([5, 1, 2, 3], [7, 5, 9], [-1, 0, 0, 0], 1, [2], [5, 2]),
    ([5, 1, 2, 3], [5, 7, 9], [-1, 0, 0, 0], 1, [1], [5, 1]),
    ([4, 1, 2, 3], [5, 7, 9], [-1, 0, 0, 0], 0, [], [4]),
    # duplicate sibling tokens: the lowest index wins
    ([5, 1, 2], [5, 5], [-1, 0, 0], 1, [1], [5, 1]),
    # two branches; the walk takes the second branch and then its child
    ([3, 8, 9, 6, 1], [8, 3, 9, 4], [-1, 0, 0, 2, 2], 2, [2, 3], [3, 9, 6]),
    # the first branch matches at depth 1 only; its sibling subtree is never visited
    ([3, 9, 0, 0, 0], [3, 7, 9, 9], [-1, 0, 1, 0, 3], 1, [1], [3, 9]),
    # a full chain match
    ([1, 2, 3, 4], [1, 2, 3], [-1, 0, 1, 2], 3, [1, 2, 3], [1, 2, 3, 4]),
    # the empty tree
    ([6], [], [-1], 0, [], [6]),
])
def test_tree_accept_hand_cases(g, toks, par, acc, path, emit):
    r = _accept1(g, toks, par)
    assert r["status"][0] == 0
    assert r["accept_len"][0] == acc and r["n_emit"][0] == acc + 1
    assert list(r["path"][0, :acc]) == path and (r["path"][0, acc:] == -1).all()
    assert list(r["emit"][0, :acc + 1]) == emit and (r["emit"][0, acc + 1:] == -1).all()
    assert r["next_tok"][0] == emit[-1] and r["pos_out"][0] == 10 + acc + 1


def _brute_accept(g, toks, par, mp):
    """Stated over all nodes at once: node v is reachable when every node u on its
    path maps to the target of u's parent and is the lowest-index child of that
    parent with its mapped token; the accepted node is the deepest reachable one."""
    k = len(toks)
    best = 0
    dep = _depths(par)
    for v in range(1, k + 1):
        ok = True
        for u in _path(par, v):
            first = min(c for c in range(1, k + 1) if par[c] == par[u] and mp(toks[c - 1]) == mp(toks[u - 1]))
            if mp(toks[u - 1]) != g[par[u]] or first != u:
                ok = False
        if ok and dep[v] > dep[best]:
            best = v
    return _path(par, best)


def test_tree_accept_matches_brute_force_random():
    rng = np.random.default_rng(21)
    B, kmax, V, nd = 64, 12, 9, 12
    d2t = rng.integers(0, V, nd).astype(np.int32)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    parent = np.zeros((B, kmax + 1), np.int32)
    drafts = rng.integers(0, nd, (B, kmax)).astype(np.int32)
    for s in range(B):
        parent[s, :k[s] + 1] = _random_parents(rng, int(k[s]), 0.4)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    # bias the targets towards the drafts so long paths occur
    off = np.concatenate([[0], np.cumsum(k + 1)[:-1]])
    for s in range(B):
        for c in range(1, k[s] + 1):
            if rng.uniform() < 0.6:
                g[off[s] + parent[s, c]] = d2t[drafts[s, c - 1]]
    pos = rng.integers(0, 1000, B).astype(np.int32)
    r = oracle.tree_accept(g, drafts, kmax, k, parent, d2t, nd, V, B, R, pos)
    assert (r["status"] == 0).all()
    lens = []
    for s in range(B):
        gs = g[off[s]:off[s] + k[s] + 1]
        p = _brute_accept(gs, list(drafts[s, :k[s]]), list(parent[s, :k[s] + 1]), lambda t: int(d2t[t]))
        a = len(p)
        lens.append(a)
        assert r["accept_len"][s] == a and list(r["path"][s, :a]) == p
        last = p[-1] if p else 0
        assert list(r["emit"][s, :a + 1]) == [int(d2t[drafts[s, u - 1]]) for u in p] + [int(gs[last])]
        assert r["pos_out"][s] == pos[s] + a + 1 and r["next_tok"][s] == gs[last]
    assert max(lens) >= 3 and min(lens) == 0


def test_chain_tree_accept_equals_greedy_accept():
    rng = np.random.default_rng(22)
    B, kmax, V = 40, 7, 6
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    drafts = rng.integers(0, V, (B, kmax)).astype(np.int32)
    pos = rng.integers(0, 100, B).astype(np.int32)
    parent = np.tile(np.arange(-1, kmax, dtype=np.int32), (B, 1))
    a = oracle.tree_accept(g, drafts, kmax, k, parent, None, 0, V, B, R, pos)
    b = oracle.greedy_accept(g, drafts, kmax, k, None, 0, V, B, R, pos)
    for key in ("pos_out", "accept_len", "n_emit", "emit", "next_tok", "status"):
        np.testing.assert_array_equal(a[key], b[key])
    for s in range(B):
        assert list(a["path"][s, :a["accept_len"][s]]) == list(range(1, a["accept_len"][s] + 1))


def test_tree_accept_error_paths():
    r = _accept1([1, 2, 3], [1, 2], [-1, 0, 2])
    assert r["status"][0] == oracle.BAD_TREE and r["accept_len"][0] == -1 and r["n_emit"][0] == 0
    assert r["pos_out"][0] == 10 and (r["path"][0] == -1).all() and r["next_tok"][0] == -1
    r = _accept1([1, 2, 3], [1, 60], [-1, 0, 1])
    assert r["status"][0] == oracle.BAD_TOKEN
    r = _accept1([1, 2, 3], [1, 2], [-1, 0, 1], pos=-1)
    assert r["status"][0] == oracle.BAD_POS


# --------------------------------------------------------------------------- compaction
def test_compaction_equals_contiguous_append_of_the_path():
    """After the walk, the pool equals the one where the accepted path's rows had been
    appended as a chain at pos + 1..: slots 0..pos + a hold the same K/V, and the
    pages no row touched are unchanged."""
    x, parent, kmax = _tree_inputs(23, B=4, k=(4, 9), chain_bias=0.4)
    out, kp, vp, off, st = _run_tree(x, parent, kmax)
    rng = np.random.default_rng(5)
    B = x["B"]
    path = np.full((B, kmax), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for s in range(B):
        # pick a random node; its path is the accepted path
        v = int(rng.integers(0, x["k"][s] + 1))
        p = _path(parent[s], v)
        acc[s] = len(p)
        path[s, :len(p)] = p
    assert acc.max() >= 2
    kc, vc = kp.copy(), vp.copy()
    oracle.kv_compact(kc, vc, x["pt"], x["max_pages"], x["pos"], path, acc, kmax, st, B, x["Hkv"], x["D"])
    Kc, Vc = PL.unpack(kc, PL.k_offsets(x["D"])), PL.unpack(vc, PL.v_offsets(x["D"]))
    Kt, Vt = PL.unpack(kp, PL.k_offsets(x["D"])), PL.unpack(vp, PL.v_offsets(x["D"]))
    K0, V0 = Kt.copy(), Vt.copy()
    for s in range(B):
        P = int(x["pos"][s])
        chain = [0] + list(path[s, :acc[s]])
        for d, u in enumerate(chain):
            slot = P + d
            page = x["pt"][s, slot // 16]
            K0[page, :, slot % 16] = x["k_new"][off[s] + u]
            V0[page, :, slot % 16] = x["v_new"][off[s] + u]
    np.testing.assert_array_equal(Kc, K0)
    np.testing.assert_array_equal(Vc, V0)


# --------------------------------------------------------------------------- lossless
N_NEW = 64


@pytest.fixture(scope="module")
def toy():
    m = ToyLM(seed=0)
    prompt = list(np.random.default_rng(1).integers(0, m.V, 20))
    ref = m.generate_ar(prompt, N_NEW + 16)
    return m, prompt, ref


@pytest.mark.parametrize("shape", ["star", "trie", "deep"])
def test_tree_stream_equals_one_row_greedy(toy, shape):
    m, prompt, ref = toy
    rng = np.random.default_rng(8)

    def drafter(out):
        n = len(out)
        true = ref[n:n + 8]
        true = true + [0] * (8 - len(true))
        wrong = lambda t: int((t + 1 + rng.integers(0, m.V - 1)) % m.V)
        if shape == "star":      # depth 1: the true token among C = 4 children, at a random rank
            kids = [wrong(true[0]) for _ in range(4)]
            if rng.uniform() < 0.8:
                kids[int(rng.integers(0, 4))] = true[0]
            return [0] * 4, kids
        par, toks = [], []
        # a chain along the truth with corruption, plus side branches hanging off it
        depth = 6 if shape == "deep" else 3
        spine = [0]
        for d in range(depth):
            par.append(spine[-1])
            toks.append(true[d] if rng.uniform() < 0.75 else wrong(true[d]))
            spine.append(len(toks))
            if shape == "trie" and rng.uniform() < 0.7:      # a sibling of the spine node
                par.append(spine[-2])
                toks.append(true[d] if toks[-1] != true[d] else wrong(true[d]))
        return par, toks

    out, hist = m.generate_tree(prompt, N_NEW, drafter)
    assert out == ref[:N_NEW]
    assert max(hist) >= 1
    if shape != "star":
        assert max(hist) >= 3
