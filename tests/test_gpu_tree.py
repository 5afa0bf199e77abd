"""GPU parity of the tree (trie / star) entry points against the CPU oracle.

DSSD fast.py _set_rows / _tree_cycle / _star_cycle: rows are the nodes of a draft
tree in creation order; node j appends at slot pos + j and attends to slots 0..pos
plus the slots of its own path; the acceptance walk follows the child whose token is
the current node's greedy token; the accepted path's K/V moves to slots pos + 1...

Bars: tree attention within |err| <= 2e-2 + 1e-2 |ref| of the oracle, the K/V append
and the compaction bit-exact, the acceptance walk bit-exact; every tree row gives the
bytes of its one-row decode after compaction (so a chain-shaped tree gives the chain
entry point's bytes, and a row's bytes do not depend on the nodes outside its path).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import (assert_close, bits, gpu_attn, gpu_attn_tree, gpu_tree_accept, i32, oracle_attn,
                           oracle_attn_tree)
from tests.test_gpu_kernels import _wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


TREE_CASES = [
    # name, B, k range, ctx range, Hq, Hkv, D, max_pages
    _wl("t64", 3, 3, 9, 1, 700, 4, 1, 64, 64),
    _wl("t128", 4, 5, 15, 200, 1100, 32, 8, 128, 80),      # G * (kmax + 1) = 64
    _wl("t256", 2, 6, 12, 500, 900, 16, 2, 256, 64),       # G * (kmax + 1) = 104
    _wl("tbig", 2, 100, 127, 30, 300, 1, 1, 64, 32),       # 128 nodes: every mask word, two row groups
    _wl("tdeep", 2, 40, 63, 300, 900, 32, 8, 128, 64),     # G * (kmax + 1) = 256: four row groups
]


def _tree_case(wl, seed, shape):
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    parent = synth.make_parents(x.k, seed, wl.name, shape, kmax=wl.kmax)
    return x, parent


@pytest.mark.parametrize("wl", TREE_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("shape", ["trie", "star", "random"])
@pytest.mark.parametrize("split", [0, 64, 1024])   # 1024: pool read with non-temporal loads
def test_tree_attention_parity(dev, wl, shape, split):
    print(f"tree attention {wl.name} {shape} split={split}", flush=True)
    x, parent = _tree_case(wl, 0, shape)
    out, kp, vp, st = gpu_attn_tree(x, parent, dev, kv_split_tokens=split)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn_tree(x, parent)
    assert (st == 0).all() and (st_ref == 0).all()
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, f"tree attention {wl.name} {shape}")


def test_b16tree_attention_sampled(dev):
    """The 16-node tree workload at full size (context up to 4096, 32q / 8kv, D = 128):
    a third of the sequences against the oracle."""
    x = synth.make_verify_inputs("b16tree", seed=0, with_lm_head=False)
    parent = synth.make_parents(x.k, 0, "b16tree", "trie")
    out, kp, vp, st = gpu_attn_tree(x, parent, dev)
    assert (st == 0).all()
    seqs = [0, 5, 10, 15, 3]
    rows, ref, _, _, st_ref = oracle_attn_tree(x, parent, seqs=seqs)
    assert (st_ref == 0).all()
    assert_close(out.float().cpu().numpy()[rows], ref, "b16tree attention")


@pytest.mark.parametrize("wl", TREE_CASES[:3], ids=lambda w: w.name)
@pytest.mark.parametrize("split", [0, 64, 1024])
def test_chain_tree_gives_chain_bytes(dev, wl, split):
    x = synth.make_verify_inputs(wl, seed=1, with_lm_head=False)
    parent = synth.make_parents(x.k, 1, wl.name, "chain", kmax=wl.kmax)
    out_t, kp_t, vp_t, st_t = gpu_attn_tree(x, parent, dev, kv_split_tokens=split)
    out_c, kp_c, vp_c, st_c = gpu_attn(x, dev, kv_split_tokens=split, kmax=wl.kmax)
    assert (st_t == 0).all() and (st_c == 0).all()
    assert torch.equal(out_t.view(torch.int16), out_c.view(torch.int16))
    assert torch.equal(kp_t.view(torch.int16), kp_c.view(torch.int16))
    assert torch.equal(vp_t.view(torch.int16), vp_c.view(torch.int16))


def _paths(parent, ks):
    """Each node's path from the root, in depth order."""
    paths = []
    for j in range(ks + 1):
        p, u = [], j
        while u != -1:
            p.append(u)
            u = int(parent[u])
        paths.append(p[::-1])
    return paths


def _assert_rows_equal(out, ref, x, parent, what):
    """Bytes equal; otherwise names the first differing rows (sequence, node, depth)."""
    a, b = out.view(torch.int16).cpu().numpy(), ref.view(torch.int16).cpu().numpy()
    bad = np.nonzero((a != b).reshape(a.shape[0], -1).any(axis=1))[0]
    if len(bad):
        off = np.concatenate([[0], np.cumsum(x.k + 1)])
        desc = []
        for r in bad[:8]:
            s = int(np.searchsorted(off, r, side="right") - 1)
            j = int(r - off[s])
            d = len(_paths(parent[s], int(x.k[s]))[j]) - 1
            desc.append(f"seq {s} node {j} depth {d} pos {int(x.pos[s])}")
        raise AssertionError(f"{what}: {len(bad)} of {a.shape[0]} rows differ: " + "; ".join(desc))


def _one_row_decodes(x, parent, dev, split):
    """Every tree row as its one-row decode once its path is compacted: for node j of
    sequence s at depth d, a one-row sequence whose slots pos..pos + d - 1 hold the
    path's nodes 0 = a_0, .., a_{d-1} (appended by a chain call) and whose row is node
    j's query at position pos + d with node j's K/V as its new row. Each such sequence
    gets its own copies of the pages from pos on. Returns the rows' bytes [R, Hq, D]."""
    B = len(x.pos)
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    n0 = x.k_pool.shape[0]
    src_pages, tables, ent = [], [], []
    for s in range(B):
        P0 = int(x.pos[s])
        for j, path in enumerate(_paths(parent[s], int(x.k[s]))):
            d = len(path) - 1
            row = x.page_table[s].copy()
            for pg in range(P0 // 16, (P0 + d) // 16 + 1):
                src_pages.append(int(row[pg]))
                row[pg] = n0 + len(src_pages) - 1
            tables.append(row)
            ent.append((s, P0, d, [int(off[s] + a) for a in path]))
    src = torch.tensor(src_pages, dtype=torch.long)
    kp = torch.cat([x.k_pool, x.k_pool[src]]).to(dev)
    vp = torch.cat([x.v_pool, x.v_pool[src]]).to(dev)
    tables = np.stack(tables).astype(np.int32)
    # the path's nodes above the row go to slots pos .. pos + d - 1
    pre = [i for i, e in enumerate(ent) if e[2] >= 1]
    if pre:
        kk = np.array([ent[i][2] - 1 for i in pre], np.int32)
        rows = torch.tensor([r for i in pre for r in ent[i][3][:-1]], dtype=torch.long)
        q0 = torch.zeros((len(rows), x.wl.Hq, x.wl.D), dtype=torch.bfloat16)
        _, kp, vp, st = gpu_attn(x, dev, kv_split_tokens=split, pos=np.array([ent[i][1] for i in pre], np.int32),
                                 k=kk, page_table=tables[pre], k_pool=kp, v_pool=vp, q=q0, k_new=x.k_new[rows],
                                 v_new=x.v_new[rows], kmax=int(kk.max()))
        assert (st == 0).all()
    last = torch.tensor([e[3][-1] for e in ent], dtype=torch.long)
    out, _, _, st = gpu_attn(x, dev, kv_split_tokens=split, pos=np.array([e[1] + e[2] for e in ent], np.int32),
                             k=np.zeros(len(ent), np.int32), page_table=tables, k_pool=kp, v_pool=vp, q=x.q[last],
                             k_new=x.k_new[last], v_new=x.v_new[last], kmax=0)
    assert (st == 0).all()
    return out


@pytest.mark.parametrize("wl", TREE_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("shape", ["trie", "star", "random"])
@pytest.mark.parametrize("split", [0, 64])
def test_tree_row_is_its_one_row_decode(dev, wl, shape, split):
    """DSSD fast.py _attention: a tree row attends to its exact path, so its bytes are
    those of the one-row decode at pos + depth after the path is compacted."""
    print(f"tree row = one-row decode {wl.name} {shape} split={split}", flush=True)
    x, parent = _tree_case(wl, 5, shape)
    out, _, _, st = gpu_attn_tree(x, parent, dev, kv_split_tokens=split)
    assert (st == 0).all()
    ref = _one_row_decodes(x, parent, dev, split)
    _assert_rows_equal(out, ref, x, parent, f"{wl.name} {shape}")


def test_tree_rows_at_the_lds_limit(dev):
    """D = 256 with kmax = 93: the tile, K and V of 93 new rows and the node tables take
    163,056 of the workgroup's 163,840 bytes of LDS; every row is still its one-row
    decode, and one more draft is refused before launch."""
    import greedy_draft_verify_amd as gdv
    wl = _wl("tlds", 2, 80, 93, 100, 400, 2, 2, 256, 40)
    x, parent = _tree_case(wl, 6, "random")
    assert parent.shape[1] == 94
    out, _, _, st = gpu_attn_tree(x, parent, dev)
    assert (st == 0).all()
    ref = _one_row_decodes(x, parent, dev, 0)
    _assert_rows_equal(out, ref, x, parent, "tlds")
    wide = np.concatenate([parent, np.full((len(x.k), 1), -1, np.int32)], 1)   # kmax = 94
    with pytest.raises(gdv.SpecError, match="LDS"):
        gpu_attn_tree(x, wide, dev)


def test_b16tree_rows_are_their_one_row_decodes(dev):
    """The 16-node tree workload at full size, every row of every sequence."""
    x = synth.make_verify_inputs("b16tree", seed=0, with_lm_head=False)
    parent = synth.make_parents(x.k, 0, "b16tree", "trie")
    out, _, _, st = gpu_attn_tree(x, parent, dev)
    assert (st == 0).all()
    ref = _one_row_decodes(x, parent, dev, 0)
    _assert_rows_equal(out, ref, x, parent, "b16tree")


@pytest.mark.parametrize("wl", [TREE_CASES[1], TREE_CASES[3]], ids=lambda w: w.name)
def test_tree_row_ignores_nodes_off_its_path(dev, wl):
    """Re-drawing the K/V of every node outside node j's path leaves the bytes of j and of
    its ancestors unchanged."""
    x, parent = _tree_case(wl, 2, "random")
    out0, *_ = gpu_attn_tree(x, parent, dev)
    rng = np.random.default_rng(4)
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    kn, vn = x.k_new.clone(), x.v_new.clone()
    keep = []
    for s in range(len(x.k)):
        j = int(rng.integers(1, x.k[s] + 1))
        on = {0}
        u = j
        while u != 0:
            on.add(u)
            u = int(parent[s, u])
        keep += [int(off[s] + u) for u in sorted(on)]
        for u in range(x.k[s] + 1):
            if u not in on:
                kn[off[s] + u] = torch.randn_like(kn[off[s] + u], dtype=torch.float32).to(torch.bfloat16)
                vn[off[s] + u] = torch.randn_like(vn[off[s] + u], dtype=torch.float32).to(torch.bfloat16)
    y = synth.VerifyInputs(x.wl, x.pos, x.k, x.R, x.page_table, x.n_pages, x.q, kn, vn, x.k_pool, x.v_pool,
                           x.hidden, x.w, x.d2t)
    out1, *_ = gpu_attn_tree(y, parent, dev)
    keep = torch.tensor(keep, device=dev)
    assert torch.equal(out0[keep].view(torch.int16), out1[keep].view(torch.int16))
    assert not torch.equal(out0.view(torch.int16), out1.view(torch.int16))


def test_tree_attention_flags_bad_parents(dev):
    wl = TREE_CASES[1]
    x, parent = _tree_case(wl, 3, "trie")
    parent = parent.copy()
    parent[1, 3] = 3            # not before its node
    parent[2, 0] = 0            # root must have parent -1
    out, kp, vp, st = gpu_attn_tree(x, parent, dev)
    assert list(st) == [0, oracle.BAD_TREE, oracle.BAD_TREE, 0]
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    o = out.float().cpu().numpy()
    for s in (1, 2):
        assert np.isnan(o[off[s]:off[s + 1]]).all()
    # flagged sequences write nothing into the pool: compare with the oracle's pools,
    # where flagged sequences are skipped the same way
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn_tree(x, parent)
    assert list(st_ref) == list(st)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    good = np.concatenate([np.arange(off[s], off[s + 1]) for s in (0, 3)])
    assert_close(o[good], ref[good], "tree attention next to flagged sequences")


# --------------------------------------------------------------------------- acceptance
def _accept_inputs(seed, B, kmax, shape, V=500, n_d2t=0, k_fixed=False, p_corrupt=0.3):
    rng = np.random.default_rng(seed)
    k = np.full(B, kmax, np.int32) if k_fixed else rng.integers(0, kmax + 1, B).astype(np.int32)
    parent = synth.make_parents(k, seed, "b16tree", shape, kmax=kmax)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    target = [g[off[s]:off[s + 1]] for s in range(B)]
    wl = synth.VerifyWorkload("acc", B=B, k=None, k_lo=0, k_hi=kmax, ctx_lo=0, ctx_hi=0, Hq=1, Hkv=1, D=64, H=1,
                              V=V, max_pages=1, p_corrupt=(p_corrupt, p_corrupt))
    drafts = synth.make_tree_drafts(wl, k, parent, target, seed)
    d2t = None
    if n_d2t:
        # drafts become draft-vocabulary ids of a map that reaches every target id
        d2t = (rng.permutation(n_d2t) % V).astype(np.int32)
        inv = {}
        for i, t in enumerate(d2t):
            inv.setdefault(int(t), i)
        mapped = np.vectorize(lambda t: inv[int(t)], otypes=[np.int32])(np.maximum(drafts, 0))
        drafts = np.where(drafts >= 0, mapped, -1).astype(np.int32)
    pos = rng.integers(0, 100000, B).astype(np.int32)
    return g, drafts, k, parent, d2t, V, pos, R


def _oracle_accept(g, drafts, k, parent, d2t, V, pos, R):
    B, kmax = drafts.shape
    return oracle.tree_accept(g, drafts, kmax, k, parent, d2t, 0 if d2t is None else len(d2t), V, B, R, pos)


def _assert_tree_accept_equal(got, ref, what):
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "path"):
        assert np.array_equal(got[key], ref[key]), f"{what}: {key}\ngpu {got[key]}\nref {ref[key]}"


@pytest.mark.parametrize("B,kmax,shape,n_d2t", [(16, 15, "trie", 0), (64, 15, "star", 0), (64, 31, "random", 0),
                                                (200, 127, "trie", 0), (4096, 15, "trie", 0),
                                                (32, 63, "trie", 700), (8192, 4, "random", 0)])
def test_tree_accept_parity(dev, B, kmax, shape, n_d2t):
    print(f"tree accept B={B} kmax={kmax} {shape} d2t={n_d2t}", flush=True)
    args = _accept_inputs(B * 7 + kmax, B, kmax, shape, n_d2t=n_d2t)
    ref = _oracle_accept(*args)
    got = gpu_tree_accept(*args[:-1], dev)
    _assert_tree_accept_equal(got, ref, f"tree accept B={B} kmax={kmax} {shape}")
    assert (ref["status"] == 0).all()
    assert ref["accept_len"].max() >= (1 if shape == "star" else min(kmax, 3))


def test_tree_accept_deep_paths_and_duplicates(dev):
    """Full 127-deep chains accepted to the end (both lane halves of the walk), and
    duplicate sibling tokens (the lowest index wins)."""
    B, kmax = 8, 127
    args = list(_accept_inputs(99, B, kmax, "chain", k_fixed=True, p_corrupt=0.0))
    ref = _oracle_accept(*args)
    assert (ref["accept_len"] == kmax).all()
    _assert_tree_accept_equal(gpu_tree_accept(*args[:-1], dev), ref, "deep chains")
    # a star of identical children: node 1 wins whenever the token matches
    g, drafts, k, parent, d2t, V, pos, R = _accept_inputs(5, 64, 8, "star", k_fixed=True, p_corrupt=0.0)
    drafts[:, :] = drafts[:, :1]
    ref = _oracle_accept(g, drafts, k, parent, d2t, V, pos, R)
    assert (ref["path"][:, 0] == 1).all()
    _assert_tree_accept_equal(gpu_tree_accept(g, drafts, k, parent, d2t, V, pos, dev), ref, "duplicate siblings")


def test_tree_accept_error_paths(dev):
    g, drafts, k, parent, d2t, V, pos, R = _accept_inputs(3, 6, 7, "trie", k_fixed=True)
    parent = parent.copy()
    drafts = drafts.copy()
    pos = pos.copy()
    parent[0, 2] = 5                 # after its node
    parent[1, 0] = 3                 # root
    drafts[2, 3] = V + 4             # token outside the vocabulary
    pos[3] = -1
    parent[4, 1] = -1                # a node without a parent
    ref = _oracle_accept(g, drafts, k, parent, d2t, V, pos, R)
    assert list(ref["status"]) == [oracle.BAD_TREE, oracle.BAD_TREE, oracle.BAD_TOKEN, oracle.BAD_POS,
                                   oracle.BAD_TREE, 0]
    _assert_tree_accept_equal(gpu_tree_accept(g, drafts, k, parent, d2t, V, pos, dev), ref, "error paths")
    # packing that does not add up flags every sequence
    ref = _oracle_accept(g, drafts, k, parent, d2t, V, pos, R + 1)
    got = gpu_tree_accept(np.concatenate([g, [0]]), drafts, k, parent, d2t, V, pos, dev)
    assert (got["status"] & oracle.BAD_ROWS).all()
    _assert_tree_accept_equal(got, ref, "bad packing")


# --------------------------------------------------------------------------- compaction
@pytest.mark.parametrize("wl", [TREE_CASES[0], TREE_CASES[1], TREE_CASES[2], TREE_CASES[3]],
                         ids=lambda w: w.name)
def test_kv_compact_parity(dev, wl):
    import greedy_draft_verify_amd as gdv
    x, parent = _tree_case(wl, 6, "random")
    B, kmax = len(x.k), wl.kmax
    rng = np.random.default_rng(8)
    path = np.full((B, kmax), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for s in range(B):
        j = int(rng.integers(0, x.k[s] + 1)) if s else int(x.k[s])   # sequence 0: the deepest-numbered node
        p = []
        while j != 0:
            p.append(j)
            j = int(parent[s, j])
        p = p[::-1]
        acc[s] = len(p)
        path[s, :len(p)] = p
    st_in = np.zeros(B, np.int32)
    if B > 2:
        st_in[2] = oracle.BAD_PAGE         # flagged upstream: must not move
    kp = x.k_pool.to(dev).clone()
    vp = x.v_pool.to(dev).clone()
    st = i32(st_in, dev)
    gdv.spec_kv_compact(kp, vp, i32(x.page_table, dev), i32(x.pos, dev), i32(path, dev), i32(acc, dev), st)
    torch.cuda.synchronize()
    kp_ref, vp_ref = bits(x.k_pool).copy(), bits(x.v_pool).copy()
    oracle.kv_compact(kp_ref, vp_ref, x.page_table, x.page_table.shape[1], x.pos, path, acc, kmax, st_in, B,
                      wl.Hkv, wl.D)
    assert list(st.cpu().numpy()) == list(st_in)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert acc.max() >= 2


def test_kv_compact_rejects_bad_paths(dev):
    import greedy_draft_verify_amd as gdv
    wl = TREE_CASES[1]
    x, parent = _tree_case(wl, 7, "trie")
    B, kmax = len(x.k), wl.kmax
    path = np.full((B, kmax), -1, np.int32)
    acc = np.array([2, 2, 3, 1], np.int32)
    path[0, :2] = [3, 3]           # not increasing
    path[1, :2] = [1, kmax + 1]    # past kmax
    path[2, :3] = [2, 4, 5]        # fine (k >= 5 in this workload)
    path[3, :1] = [1]              # fine, and equal to its destination: nothing moves
    kp = x.k_pool.to(dev).clone()
    vp = x.v_pool.to(dev).clone()
    st = i32(np.zeros(B), dev)
    gdv.spec_kv_compact(kp, vp, i32(x.page_table, dev), i32(x.pos, dev), i32(path, dev), i32(acc, dev), st)
    torch.cuda.synchronize()
    assert list(st.cpu().numpy()) == [oracle.BAD_TREE, oracle.BAD_TREE, 0, 0]
    kp_ref, vp_ref = bits(x.k_pool).copy(), bits(x.v_pool).copy()
    oracle.kv_compact(kp_ref, vp_ref, x.page_table, x.page_table.shape[1], x.pos, path, acc, kmax,
                      np.array([1, 1, 0, 0], np.int32), B, wl.Hkv, wl.D)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)


@pytest.mark.parametrize("tree", [False, True])
def test_attention_status_combinations_match_the_oracle(dev, tree):
    """Each check reports on its own, as the oracle does: an undefined packing flags
    every sequence BAD_ROWS and the page, position and parent checks still add their
    bits to it; a flagged sequence writes nothing into the pool and leaves its rows."""
    wl = TREE_CASES[1] if tree else _wl("cmb", 5, 1, 3, 40, 200, 8, 2, 64, 32)
    x, parent = _tree_case(wl, 6, "trie") if tree else (synth.make_verify_inputs(wl, seed=6, with_lm_head=False), None)
    B = len(x.pos)
    pt = x.page_table.copy()
    pt[1, 1] = -4                            # a page id out of range
    pos = x.pos.copy()
    pos[2] = -1                              # a negative position
    if tree:
        parent = parent.copy()
        parent[1, 1] = 5                     # a parent after its node (with the bad page)
        parent[3, 0] = 2                     # the root's parent must be -1
    kmax = wl.kmax
    for k_use in (x.k, x.k + np.eye(B, dtype=np.int32)[B - 1]):     # rows that add up, then rows that do not
        R = x.R
        y = synth.VerifyInputs(x.wl, pos, k_use, R, pt, x.n_pages, x.q, x.k_new, x.v_new, x.k_pool, x.v_pool,
                               x.hidden, x.w, x.d2t)
        if tree:
            out, kp, vp, st = gpu_attn_tree(y, parent, dev)
        else:
            out, kp, vp, st = gpu_attn(y, dev, kmax=kmax)
        _, st_ref = oracle.validate(pt, pt.shape[1], x.n_pages, pos, k_use, kmax, B, R)
        if tree:
            oracle.validate_tree(parent, kmax, k_use, B, st_ref)
        assert np.array_equal(st, st_ref), (st, st_ref)
        assert (st != 0).sum() >= 2
        flagged = np.flatnonzero(st != 0)
        if (st == 0).any():
            off = np.concatenate([[0], np.cumsum(k_use + 1)])
            o = out.float().cpu().numpy()
            for s in flagged:
                assert np.isnan(o[off[s]:off[s + 1]]).all()
            good = [s for s in range(B) if st[s] == 0]
            if tree:
                ref_k, ref_v = oracle_attn_tree(y, parent, seqs=good)[2:4]
            else:
                ref_k, ref_v = oracle_attn(y, seqs=good)[2:4]
            assert np.array_equal(bits(kp), ref_k) and np.array_equal(bits(vp), ref_v)
        else:
            assert np.isnan(out.float().cpu().numpy()).all()
            assert np.array_equal(bits(kp), bits(x.k_pool)) and np.array_equal(bits(vp), bits(x.v_pool))


@pytest.mark.parametrize("tree", [False, True])
def test_attention_ignores_workspace_contents(dev, tree):
    """The merge reads only partials this call wrote: a workspace full of 0xFF bytes (NaN
    partials) gives the bytes of a zeroed one, at the full b16 sizes."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16tree" if tree else "b16k4", seed=0, device=dev, with_lm_head=False)
    wl = x.wl
    B = len(x.pos)
    pt, pos, k = (torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev) for a in (x.page_table, x.pos, x.k))
    parent = torch.from_numpy(synth.make_parents(x.k, 0, "b16tree", "trie")).to(dev) if tree else None
    if tree:
        nbytes = gdv.verify_attn_tree_workspace_bytes(B, x.R, wl.Hq, wl.Hkv, wl.D, x.page_table.shape[1], wl.kmax)
    else:
        nbytes = gdv.verify_attn_workspace_bytes(B, x.R, wl.Hq, wl.Hkv, wl.D, x.page_table.shape[1])
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=dev)
        kp, vp = x.k_pool.clone(), x.v_pool.clone()
        out = torch.full((x.R, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
        st = torch.full((B,), -7, dtype=torch.int32, device=dev)
        if tree:
            gdv.spec_verify_attn_tree(x.q, x.k_new, x.v_new, kp, vp, pt, pos, k, parent, x.scale, out, st,
                                      workspace_buf=ws)
        else:
            gdv.spec_verify_attn(x.q, x.k_new, x.v_new, kp, vp, pt, pos, k, wl.kmax, x.scale, out, st,
                                 workspace_buf=ws)
        torch.cuda.synchronize()
        assert (st == 0).all()
        assert not torch.isnan(out.float()).any()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


# --------------------------------------------------------------------------- new-row slots
POISON_CASES = [_wl("pchain", 24, 3, 6, 200, 700, 8, 2, 128, 48), _wl("ptree", 16, 15, 15, 200, 700, 8, 2, 128, 48),
                _wl("pd64", 12, 5, 9, 100, 500, 4, 1, 64, 40), _wl("pd256", 8, 7, 13, 100, 400, 8, 2, 256, 32),
                "b16k4", "b16tree"]


def _poison_new_row_slots(x):
    """Sets the pool's K and V at positions pos .. pos + k of every sequence (the slots
    the call appends to) to 4096."""
    from tests.pool_layout import k_offsets, v_offsets
    kb, vb = bits(x.k_pool).copy(), bits(x.v_pool).copy()
    big = np.uint16(0x4580)     # 4096.0 in bf16
    ko, vo = k_offsets(x.wl.D), v_offsets(x.wl.D)
    for s in range(len(x.pos)):
        for p in range(int(x.pos[s]), int(x.pos[s]) + int(x.k[s]) + 1):
            page, t = int(x.page_table[s, p // 16]), p % 16
            kb[page, :, ko[t]] = big
            vb[page, :, vo[t]] = big
    x.k_pool = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16)
    x.v_pool = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("wl", POISON_CASES, ids=lambda w: w if isinstance(w, str) else w.name)
def test_new_row_slots_never_keep_old_pool_values(dev, wl):
    """The pool's slots at positions pos .. pos + k (the rows being verified) hold 4096
    before the call; the kernel must read the new rows there (the oracle appends them
    first), so a new-row value lost in the tile's LDS copy shows as an error of
    hundreds. Repeated calls must give identical bytes (at the b16 sizes the oracle
    checks four sequences, over 30 calls: such a loss depends on the waves' timing)."""
    full = isinstance(wl, str)
    x = synth.make_verify_inputs(wl, seed=5 if not full else 0, device="cpu", with_lm_head=False)
    tree = (wl if full else wl.name) in ("ptree", "b16tree")
    _poison_new_row_slots(x)
    parent = synth.make_parents(x.k, 0 if full else 5, "b16tree", "trie") if tree else None
    seqs = [0, 5, 11, 15] if full else None
    reps = 30 if full else 6
    print(f"[poison] {x.wl.name}: B={len(x.pos)} D={x.wl.D} tree={tree}", flush=True)
    if tree:
        rows, ref, _, _, st = oracle_attn_tree(x, parent, seqs=seqs)
    else:
        rows, ref, _, _, st = oracle_attn(x, seqs=seqs)
    assert (st == 0).all()
    # device-resident inputs: the calls run back to back, as in a decode loop
    for name in ("q", "k_new", "v_new", "k_pool", "v_pool"):
        setattr(x, name, getattr(x, name).to(dev))
    first = None
    for rep in range(reps):
        out, _, _, status = gpu_attn_tree(x, parent, dev) if tree else gpu_attn(x, dev)
        assert (status == 0).all()
        assert_close(out.float().cpu().numpy()[rows], ref, f"{x.wl.name} call {rep}")
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"{x.wl.name}: call {rep} differs"
