"""Seeded random shapes against the oracle, beside the hand-picked cases: head dims,
query/kv head ratios, batch sizes, ragged k, positions from 0 up, split sizes and kmax
above the largest k for the chain and tree attention (tree shapes trie, star, random
and chain; every other seed with the new-row slots of the pool set to 4096 beforehand), row / vocabulary / hidden sizes for the lm_head and its sampling form
(support sizes and temperatures too), and batch, draft length, head count and accepted
lengths (0 up to past the draft) for the DeltaNet record / rollback and input-stash
modes. Each case prints its parameters first; the same tolerance as the other parity
tests."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import (assert_close, bits, check_argmax, gpu_attn, gpu_attn_tree, gpu_lm_head, oracle_attn,
                           oracle_attn_tree)
from tests.test_gpu_tree import _poison_new_row_slots

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SPLITS = [0, 64, 128, 192, 256, 320, 512, 1024, 2048]
# GDV_RANDOM_SCALE multiplies the number of seeds of every test here (a longer sweep)
_SCALE = max(1, int(os.environ.get("GDV_RANDOM_SCALE", "1")))


def _seeds(n):
    return range(n * _SCALE)


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _random_workload(seed, k_cap):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 6))
    k_lo = int(rng.integers(0, k_cap // 2 + 1))
    k_hi = int(rng.integers(k_lo, k_cap + 1))
    ctx_lo = int(rng.integers(0, 1500))
    ctx_hi = ctx_lo + int(rng.integers(0, 700))
    wl = synth.VerifyWorkload(f"rand{seed}", B=B, k=None, k_lo=k_lo, k_hi=k_hi, ctx_lo=ctx_lo, ctx_hi=ctx_hi,
                              Hq=G * Hkv, Hkv=Hkv, D=D, H=256, V=1000, max_pages=16, w_std=1 / 16)
    split = int(rng.choice(SPLITS))
    kmax = min(127, k_hi + int(rng.integers(0, 12)))
    return wl, split, kmax, rng


@pytest.mark.parametrize("seed", _seeds(16))
def test_attention_random_shapes(dev, seed):
    wl, split, kmax, _ = _random_workload(seed, 12)
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    if seed % 2:
        _poison_new_row_slots(x)    # a new-row value lost on the way to the tile shows as a large error
    print(f"[rand attn] seed {seed}: D={wl.D} Hq={wl.Hq} Hkv={wl.Hkv} B={len(x.pos)} pos {x.pos.tolist()} "
          f"k {x.k.tolist()} kmax {kmax} split {split}", flush=True)
    out, kp, vp, st = gpu_attn(x, dev, kv_split_tokens=split, kmax=kmax)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn(x)
    assert list(st) == list(st_ref) == [0] * len(x.pos)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, f"random attention seed {seed}")


@pytest.mark.parametrize("seed", _seeds(8))
def test_tree_attention_random_shapes(dev, seed):
    wl, split, _, rng = _random_workload(100 + seed, 20)
    shape = ["trie", "star", "random", "chain"][seed % 4]
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    if seed % 2:
        _poison_new_row_slots(x)
    parent = synth.make_parents(x.k, seed, wl.name, shape, kmax=wl.kmax)
    print(f"[rand tree] seed {seed}: D={wl.D} Hq={wl.Hq} Hkv={wl.Hkv} B={len(x.pos)} pos {x.pos.tolist()} "
          f"k {x.k.tolist()} shape {shape} split {split}", flush=True)
    out, kp, vp, st = gpu_attn_tree(x, parent, dev, kv_split_tokens=split)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn_tree(x, parent)
    assert (st == 0).all() and (st_ref == 0).all()
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, f"random tree attention seed {seed}")


@pytest.mark.parametrize("seed", _seeds(8))
def test_lm_head_random_shapes(dev, seed):
    rng = np.random.default_rng(8000 + seed)
    R = int(rng.integers(1, 400))
    H = int(rng.choice([256, 512, 768, 1024]))
    V = int(rng.integers(1, 6000))
    print(f"[rand lm_head] seed {seed}: R={R} H={H} V={V}", flush=True)
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    g, mv = gpu_lm_head(h, w, dev)
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(h), bits(w), R, H, V)
    n_undecided = check_argmax(g, mv, g_ref, t1, t2, f"random lm_head seed {seed}")
    assert n_undecided <= max(2, R // 3)


@pytest.mark.parametrize("seed", _seeds(6))
def test_lm_head_sample_random_shapes(dev, seed):
    import greedy_draft_verify_amd as gdv
    from tests.test_gpu_sampling import _check_rows, _support, gpu_sample_rows
    rng = np.random.default_rng(8500 + seed)
    R = int(rng.integers(1, 300))
    H = int(rng.choice([256, 512]))
    V = int(rng.integers(100, 5000))
    NQ = int(rng.integers(0, 9))
    T = float(rng.uniform(0.4, 1.6))
    print(f"[rand sample] seed {seed}: R={R} H={H} V={V} NQ={NQ} T={T:.3f}", flush=True)
    g = torch.Generator().manual_seed(8500 + seed)
    hidden = torch.randn((R, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, H), generator=g) / math.sqrt(H / 4)).to(torch.bfloat16)
    q_tok, q_prob = _support(rng, R, V, NQ)
    row_ctr = np.stack([rng.integers(0, 1 << 20, R), rng.integers(0, 1 << 30, R)], 1).astype(np.int32)
    key = int(rng.integers(0, 1 << 62))
    wp = gdv.spec_lm_head_pack(w.to(dev))
    got = gpu_sample_rows(hidden.to(dev), wp, V, T, q_tok, q_prob, row_ctr, key, dev)
    logits = oracle.lm_head_logits(bits(hidden), bits(w), R, H, V)
    ref = oracle.sample_rows(logits, T, q_tok, q_prob, row_ctr, key)
    # every decided row must match; at a few rows one near-tie is a large share
    _check_rows(got, ref, f"random sampling seed {seed}", min_decided=0.5)


@pytest.mark.parametrize("seed", _seeds(6))
def test_delta_random_shapes(dev, seed):
    """Record + fused rollback (mode 3) on random (B, T, heads) with L from 0 past T."""
    import greedy_draft_verify_amd as gdv
    rng = np.random.default_rng(8800 + seed)
    B, T, Hd = int(rng.integers(1, 5)), int(rng.integers(1, 40)), int(rng.integers(1, 4))
    L = rng.integers(0, T + 3, B).astype(np.int32)
    print(f"[rand delta] seed {seed}: B={B} T={T} Hd={Hd} L={L.tolist()}", flush=True)
    d = synth.make_delta_inputs(seed=8800 + seed, B=B, T=T, Hd=Hd)
    st = d.state.to(dev).clone()
    rec = torch.full((B, T, Hd, 128, 128), float("nan"), dtype=torch.float32, device=dev)
    o = torch.full((B, T, Hd, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    to = lambda t: t.to(dev)
    gdv.spec_delta_verify_rollback(gdv.DELTA_BOTH, to(d.q), to(d.k), to(d.v), to(d.a), to(d.b), 1.0, st, rec,
                                   torch.from_numpy(L).to(dev), o)
    torch.cuda.synchronize()
    rec_ref, o_ref = oracle.delta_verify(bits(d.q), bits(d.k), bits(d.v), d.a.numpy(), d.b.numpy(), 1.0,
                                         d.state.numpy(), B, T, Hd, 128, 128)
    assert_close(rec.cpu().numpy(), rec_ref, f"random delta record seed {seed}")
    assert_close(o.float().cpu().numpy(), o_ref, f"random delta output seed {seed}")
    for s in range(B):
        Ls = min(int(L[s]), T)
        # the restored state is the recorded S_L itself (the same bytes), or S_0 for L = 0
        want = d.state[s] if Ls == 0 else rec[s, Ls - 1].cpu()
        assert torch.equal(st[s].cpu(), want), f"sequence {s}, L {int(L[s])}"
    # the input-stash pair: VERIFY gives the same outputs and leaves S_0, RESCAN of the
    # committed prefix leaves exactly the restored bytes
    s4 = d.state.to(dev).clone()
    o4 = torch.full_like(o, float("nan"))
    gdv.spec_delta_verify_rollback(gdv.DELTA_VERIFY, to(d.q), to(d.k), to(d.v), to(d.a), to(d.b), 1.0, s4, None,
                                   None, o4)
    s5 = d.state.to(dev).clone()
    gdv.spec_delta_verify_rollback(gdv.DELTA_RESCAN, to(d.q), to(d.k), to(d.v), to(d.a), to(d.b), 1.0, s5, None,
                                   torch.from_numpy(L).to(dev), None)
    torch.cuda.synchronize()
    assert torch.equal(o4.view(torch.int16), o.view(torch.int16))
    assert torch.equal(s4.cpu(), d.state), "VERIFY must not modify the state"
    assert torch.equal(s5, st), "RESCAN must give the restored record's bytes"


# --------------------------------------------------------------------------- integer walks
def _walk_case(seed):
    rng = np.random.default_rng(9100 + seed)
    B = int(rng.choice([1, 2, 3, 16, 63, 64, 65, 200, 1500]))
    kmax = int(rng.choice([0, 1, 3, 7, 15, 31, 63, 64, 65, 127]))
    V = int(rng.integers(2, 3000))
    n_d2t = int(rng.choice([0, 0, V + int(rng.integers(0, 500))]))
    return rng, B, kmax, V, n_d2t


@pytest.mark.parametrize("seed", _seeds(10))
def test_greedy_accept_random_shapes(dev, seed):
    """Bit-exact acceptance (with and without a draft map, stop tokens and limits)
    on random batch, draft length and vocabulary sizes."""
    from tests.helpers import assert_accept_equal, gpu_accept
    from tests.test_gpu_stop import _case, gpu_accept_stop
    rng, B, kmax, V, n_d2t = _walk_case(seed)
    print(f"[rand accept] seed {seed}: B={B} kmax={kmax} V={V} d2t={n_d2t}", flush=True)
    g, drafts, k, d2t, R, pos, rng2 = _case(9100 + seed, B, kmax, V, p_match=float(rng.uniform(0.3, 0.95)),
                                            n_d2t=n_d2t)
    nd = 0 if d2t is None else len(d2t)
    got = gpu_accept(g, drafts, k, d2t, V, pos, dev, kmax=kmax)
    ref = oracle.greedy_accept(g, drafts, kmax, k, d2t, nd, V, B, R, pos)
    assert_accept_equal(got, ref, f"random accept seed {seed}")
    n_stop = int(rng.integers(0, 17))
    stops = [int(t) for t in rng2.choice(g, n_stop)] if n_stop else []
    remaining = rng2.integers(1, kmax + 3, B).astype(np.int32) if rng.uniform() < 0.5 else None
    got_s = gpu_accept_stop(g, drafts, k, d2t, V, stops, remaining, pos, dev)
    ref_s = oracle.greedy_accept_stop(g, drafts, kmax, k, d2t, nd, V, B, R, stops, remaining, pos)
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit", "done"):
        assert np.array_equal(got_s[key], ref_s[key]), (key, seed)


@pytest.mark.parametrize("seed", _seeds(10))
def test_tree_accept_random_shapes(dev, seed):
    """Bit-exact tree walks on random batch and tree sizes, shapes and draft maps."""
    from tests.helpers import gpu_tree_accept
    from tests.test_gpu_tree import _accept_inputs, _assert_tree_accept_equal, _oracle_accept
    rng = np.random.default_rng(9300 + seed)
    B = int(rng.choice([1, 5, 16, 64, 65, 300]))
    kmax = int(rng.choice([1, 2, 4, 15, 31, 63, 64, 100, 127]))   # the helpers size drafts for kmax >= 1
    shape = str(rng.choice(["trie", "star", "random", "chain"]))
    n_d2t = int(rng.choice([0, 0, 700]))
    print(f"[rand tree accept] seed {seed}: B={B} kmax={kmax} {shape} d2t={n_d2t}", flush=True)
    args = _accept_inputs(9300 + seed, B, kmax, shape, n_d2t=n_d2t, p_corrupt=float(rng.uniform(0.1, 0.6)))
    ref = _oracle_accept(*args)
    got = gpu_tree_accept(*args[:-1], dev)
    _assert_tree_accept_equal(got, ref, f"random tree accept seed {seed}")


@pytest.mark.parametrize("seed", _seeds(10))
def test_lm_head_argmax_accept_random_shapes(dev, seed):
    """spec_lm_head_argmax_accept gives the bytes of spec_lm_head_argmax followed by
    spec_greedy_accept on random batch, ragged k, draft map, hidden and vocabulary sizes
    (fused up to 96 rows, the two calls' kernels above), and its walk is the oracle's on
    its greedy tokens."""
    import greedy_draft_verify_amd as gdv
    from tests.test_gpu_fused import _run, _same
    rng = np.random.default_rng(9700 + seed)
    kmax = int(rng.choice([0, 1, 3, 7, 15, 31, 63, 95]))
    B = int(rng.integers(1, 41))
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    H = int(rng.choice([256, 512]))
    V = int(rng.integers(1, 6000))
    print(f"[rand argmax+accept] seed {seed}: B={B} kmax={kmax} R={R} H={H} V={V}", flush=True)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16).to(dev)
    g = torch.empty(R, dtype=torch.int32, device=dev)
    gdv.spec_lm_head_argmax(h, wp, V, g)
    g = g.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(k + 1)])
    p_match = float(rng.uniform(0.3, 0.95))
    drafts = np.zeros((B, kmax), np.int32)
    for s in range(B):
        for j in range(int(k[s])):
            drafts[s, j] = g[off[s] + j] if rng.random() < p_match else int(rng.integers(0, V))
    d2t_np = None
    if V > 1 and rng.random() < 0.4:
        # drafts in a draft vocabulary: id i stands for target d2t[i]
        d2t_np = rng.permutation(V).astype(np.int32)
        inv = np.argsort(d2t_np).astype(np.int32)
        drafts = inv[drafts]
    pos = rng.integers(0, 100000, B).astype(np.int32)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    d2t = None if d2t_np is None else t(d2t_np)
    a = _run(gdv, True, h, wp, V, t(drafts), t(k), d2t, t(pos))
    b = _run(gdv, False, h, wp, V, t(drafts), t(k), d2t, t(pos))
    _same(a, b, f"random argmax+accept seed {seed}")
    ref = oracle.greedy_accept(a["argmax"].numpy(), drafts, kmax, k, d2t_np, 0 if d2t_np is None else V, V, B, R,
                               pos)
    for n, m in (("pos_out", "pos_out"), ("accept_len", "accept_len"), ("n_emit", "n_emit"), ("emit", "emit"),
                 ("next_tok", "next_tok"), ("seq_status", "status")):
        assert np.array_equal(a[n].numpy(), ref[m]), (n, seed)
