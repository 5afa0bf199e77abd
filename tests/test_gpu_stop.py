"""GPU parity of spec_greedy_accept_stop (greedy acceptance with stop tokens and a
generation limit; oxinfer step, DSSD _commit) against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from tests.conftest import gpu_available
from tests.helpers import i32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def gpu_accept_stop(g, drafts, k, d2t, V, stops, remaining, pos, dev):
    import greedy_draft_verify_amd as gdv
    B, kmax = drafts.shape
    z = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, dn, st = z(), z(), z(), z(), z(), z()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    gdv.spec_greedy_accept_stop(i32(g, dev), i32(drafts, dev), i32(k, dev), None if d2t is None else i32(d2t, dev),
                                V, i32(np.asarray(stops, np.int32), dev),
                                None if remaining is None else i32(remaining, dev), i32(pos, dev), pos_out, acc, ne,
                                emit, nt, dn, st)
    torch.cuda.synchronize()
    return dict(pos_out=pos_out.cpu().numpy(), accept_len=acc.cpu().numpy(), n_emit=ne.cpu().numpy(),
                emit=emit.cpu().numpy(), next_tok=nt.cpu().numpy(), done=dn.cpu().numpy(), status=st.cpu().numpy())


def _case(seed, B, kmax, V, p_match=0.8, n_d2t=0):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.full((B, kmax), -1, np.int32)
    for s in range(B):
        m = rng.uniform(size=k[s]) < p_match
        drafts[s, :k[s]] = np.where(m, g[off[s]:off[s] + k[s]], rng.integers(0, V, k[s]))
    d2t = None
    if n_d2t:
        d2t = rng.permutation(n_d2t).astype(np.int32) % V
        inv = {}
        for i, t in enumerate(d2t):
            inv.setdefault(int(t), i)
        drafts = np.where(drafts >= 0, np.vectorize(lambda t: inv[int(t)], otypes=[np.int32])(np.maximum(drafts, 0)), -1).astype(np.int32)
    pos = rng.integers(0, 10000, B).astype(np.int32)
    return g, drafts, k, d2t, R, pos, rng


@pytest.mark.parametrize("B,kmax,V,n_stop,limit,n_d2t", [(16, 4, 50, 2, False, 0), (64, 6, 20, 3, True, 0),
                                                          (8192, 5, 30, 16, True, 0), (40, 200, 6, 1, True, 0),
                                                          (32, 7, 40, 2, True, 60), (100, 3, 10, 0, True, 0)])
def test_accept_stop_parity(dev, B, kmax, V, n_stop, limit, n_d2t):
    print(f"accept stop B={B} kmax={kmax} n_stop={n_stop} limit={limit}", flush=True)
    g, drafts, k, d2t, R, pos, rng = _case(B + kmax, B, kmax, V, n_d2t=n_d2t)
    # stop tokens drawn among the greedy tokens, so that rounds do stop
    stops = [int(t) for t in np.unique(rng.choice(g, 4 * n_stop))[:n_stop]] if n_stop else []
    remaining = rng.integers(1, kmax + 3, B).astype(np.int32) if limit else None
    ref = oracle.greedy_accept_stop(g, drafts, kmax, k, d2t, 0 if d2t is None else len(d2t), V, B, R, stops,
                                    remaining, pos)
    got = gpu_accept_stop(g, drafts, k, d2t, V, stops, remaining, pos, dev)
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "done"):
        assert np.array_equal(got[key], ref[key]), (key, got[key][:8], ref[key][:8])
    assert (ref["status"] == 0).all()
    if n_stop:
        assert ref["done"].any()


def test_accept_stop_error_paths(dev):
    g, drafts, k, d2t, R, pos, rng = _case(5, 12, 4, 30)
    remaining = np.full(12, 3, np.int32)
    remaining[2] = 0
    pos[3] = -1
    drafts[4, 0] = 99 if k[4] > 0 else drafts[4, 0]
    ref = oracle.greedy_accept_stop(g, drafts, 4, k, None, 0, 30, 12, R, [1, 2], remaining, pos)
    got = gpu_accept_stop(g, drafts, k, None, 30, [1, 2], remaining, pos, dev)
    assert ref["status"][2] == oracle.BAD_LIMIT and ref["status"][3] & oracle.BAD_POS
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "done"):
        assert np.array_equal(got[key], ref[key]), key
    ref = oracle.greedy_accept_stop(g, drafts, 4, k, None, 0, 30, 12, R + 1, [1, 2], remaining, pos)
    got = gpu_accept_stop(np.concatenate([g, [0]]), drafts, k, None, 30, [1, 2], remaining, pos, dev)
    assert (got["status"] & oracle.BAD_ROWS).all()
    for key in ("status", "emit", "done"):
        assert np.array_equal(got[key], ref[key]), key
