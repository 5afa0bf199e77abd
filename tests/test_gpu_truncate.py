"""GPU parity of spec_truncate_stop (the stop-token and limit rule applied in place
to an acceptance walk's outputs; oxinfer step, DSSD _commit) against the oracle's
truncation: bit-exact, for arbitrary walk outputs, for the greedy walk (where it
must equal the fused greedy-stop call), and for the tree walk with its path."""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import gpu_available
from tests.helpers import gpu_tree_accept, i32
from tests.test_gpu_tree import _accept_inputs, _oracle_accept

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KEYS = ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "done")


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def gpu_truncate(res, stops, remaining, pos_in, dev, path=None):
    """Uploads a walk's outputs, truncates them on the device, returns them on the host."""
    import greedy_draft_verify_amd as gdv
    t = {key: i32(np.ascontiguousarray(res[key], np.int32), dev)
         for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit")}
    B = t["emit"].shape[0]
    done = torch.full((B,), -9, dtype=torch.int32, device=dev)
    ph = None if path is None else i32(np.ascontiguousarray(path, np.int32), dev)
    gdv.spec_truncate_stop(i32(np.asarray(stops, np.int32), dev), None if remaining is None else i32(remaining, dev),
                           i32(pos_in, dev), t["pos_out"], t["accept_len"], t["n_emit"], t["emit"], t["next_tok"],
                           done, t["status"], path=ph)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in t.items()}
    out["done"] = done.cpu().numpy()
    if ph is not None:
        out["path"] = ph.cpu().numpy()
    return out


def _walk_outputs(seed, B, kmax, V, with_path, malformed=True):
    """Outputs shaped as a walk leaves them: a accepted, a + 1 emitted, pos_out = pos + a + 1,
    path = a strictly increasing node list; some sequences flagged by the walk, and (when
    malformed) some whose counts are no committed round."""
    rng = np.random.default_rng(seed)
    a = rng.integers(0, kmax + 1, B).astype(np.int32)
    pos = rng.integers(0, 50000, B).astype(np.int32)
    emit = np.full((B, kmax + 1), -1, np.int32)
    path = np.full((B, kmax), -1, np.int32) if with_path else None
    for s in range(B):
        emit[s, :a[s] + 1] = rng.integers(0, V, a[s] + 1)
        if with_path and a[s]:
            path[s, :a[s]] = np.sort(rng.choice(np.arange(1, kmax + 1), a[s], replace=False))
    res = dict(status=np.zeros(B, np.int32), accept_len=a.copy(), n_emit=a + 1, pos_out=pos + a + 1,
               next_tok=emit[np.arange(B), a].copy(), emit=emit)
    flagged = rng.uniform(size=B) < 0.05
    res["status"][flagged] = oracle.BAD_TOKEN
    res["accept_len"][flagged], res["n_emit"][flagged], res["next_tok"][flagged] = -1, 0, -1
    res["pos_out"][flagged] = pos[flagged]
    res["emit"][flagged] = -1
    if with_path:
        path[flagged] = -1
    if malformed:
        bad = np.flatnonzero(~flagged)[:3]
        if len(bad) == 3:
            res["n_emit"][bad[0]] = 0
            res["n_emit"][bad[1]] = kmax + 2
            res["accept_len"][bad[2]] = res["n_emit"][bad[2]] + 1
    return res, pos, path, rng


@pytest.mark.parametrize("B,kmax,V,n_stop,limit,with_path", [(16, 4, 30, 2, True, False), (300, 15, 20, 3, True, True),
                                                              (100003, 6, 40, 16, True, True),
                                                              (64, 200, 8, 1, True, False), (50, 127, 12, 2, False, True),
                                                              (40, 0, 5, 1, True, True), (77, 9, 25, 0, True, False)])
def test_truncate_parity(dev, B, kmax, V, n_stop, limit, with_path):
    print(f"truncate B={B} kmax={kmax} n_stop={n_stop} limit={limit} path={with_path}", flush=True)
    res, pos, path, rng = _walk_outputs(B + kmax, B, kmax, V, with_path)
    stops = [int(t) for t in rng.choice(V, n_stop, replace=False)] if n_stop else []
    remaining = rng.integers(0, kmax + 3, B).astype(np.int32) if limit else None
    ref = oracle.truncate_stop(res, kmax, stops, remaining, pos, path=path)
    got = gpu_truncate(res, stops, remaining, pos, dev, path=path)
    for key in KEYS + (("path",) if with_path else ()):
        assert np.array_equal(got[key], ref[key]), (key, got[key][:6], ref[key][:6])
    assert (ref["status"] == 0).any()
    if n_stop and V <= 40:
        assert ref["done"][ref["status"] == 0].any()
    again = gpu_truncate(got, stops, remaining, pos, dev, path=got.get("path"))
    for key in KEYS + (("path",) if with_path else ()):
        assert np.array_equal(again[key], got[key]), ("twice", key)


def test_truncate_after_greedy_walk_equals_the_fused_call(dev):
    """spec_greedy_accept then spec_truncate_stop == spec_greedy_accept_stop == the oracle."""
    import greedy_draft_verify_amd as gdv
    from tests.test_gpu_stop import _case, gpu_accept_stop
    B, kmax, V = 500, 6, 25
    g, drafts, k, d2t, R, pos, rng = _case(31, B, kmax, V)
    stops = [int(t) for t in np.unique(rng.choice(g, 8))[:3]]
    remaining = rng.integers(1, kmax + 3, B).astype(np.int32)
    z = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st, dn = z(), z(), z(), z(), z(), z()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    gdv.spec_greedy_accept(i32(g, dev), i32(drafts, dev), i32(k, dev), None, V, i32(pos, dev), pos_out, acc, ne,
                           emit, nt, st)
    gdv.spec_truncate_stop(i32(np.asarray(stops, np.int32), dev), i32(remaining, dev), i32(pos, dev), pos_out, acc,
                           ne, emit, nt, dn, st)
    torch.cuda.synchronize()
    got = dict(status=st, accept_len=acc, n_emit=ne, pos_out=pos_out, next_tok=nt, emit=emit, done=dn)
    got = {key: v.cpu().numpy() for key, v in got.items()}
    fused = gpu_accept_stop(g, drafts, k, None, V, stops, remaining, pos, dev)
    ref = oracle.greedy_accept_stop(g, drafts, kmax, k, None, 0, V, B, R, stops, remaining, pos)
    for key in KEYS:
        assert np.array_equal(got[key], fused[key]), key
        assert np.array_equal(got[key], ref[key]), key
    assert ref["done"].any() and (ref["status"] == 0).all()


@pytest.mark.parametrize("B,kmax,shape", [(64, 15, "trie"), (4096, 15, "trie"), (200, 127, "chain")])
def test_truncate_tree_walk(dev, B, kmax, shape):
    """The tree walk's outputs and path, truncated: only committed path nodes remain."""
    print(f"truncate tree B={B} kmax={kmax} {shape}", flush=True)
    g, drafts, k, parent, d2t, V, pos, R = _accept_inputs(B + 5 * kmax, B, kmax, shape)
    walk = _oracle_accept(g, drafts, k, parent, d2t, V, pos, R)
    got_walk = gpu_tree_accept(g, drafts, k, parent, d2t, V, pos, dev)
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "path"):
        assert np.array_equal(got_walk[key], walk[key]), key
    rng = np.random.default_rng(B)
    stops = [int(t) for t in np.unique(rng.choice(g, 12))[:4]]
    remaining = rng.integers(1, kmax + 2, B).astype(np.int32)
    ref = oracle.truncate_stop(walk, kmax, stops, remaining, pos, path=walk["path"])
    got = gpu_truncate(got_walk, stops, remaining, pos, dev, path=got_walk["path"])
    for key in KEYS + ("path",):
        assert np.array_equal(got[key], ref[key]), (key, got[key][:4], ref[key][:4])
    cut = ref["accept_len"] < walk["accept_len"]
    assert cut.any() and ref["done"].any()
    assert (ref["path"][np.arange(B), np.maximum(ref["accept_len"], 0)] == -1)[ref["accept_len"] < kmax].all()
