"""GPU parity of each entry point against the CPU oracle at sizes the oracle finishes
in seconds, spanning several tiles / splits and ragged tails, plus edge cases.

Tolerance (bf16 inputs, fp32 accumulation): |err| <= 2e-2 + 1e-2 |ref| for attention
outputs, max logits and DeltaNet states/outputs; bit-exact for KV append, argmax
(where the oracle's top-2 gap exceeds 5e-2), acceptance and all bookkeeping.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import (GAP, assert_accept_equal, assert_close, bits, check_argmax, gpu_accept,
                           gpu_attn, gpu_lm_head, i32, oracle_attn)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _wl(name, B, k_lo, k_hi, ctx_lo, ctx_hi, Hq, Hkv, D, max_pages, H=256, V=1000):
    return synth.VerifyWorkload(name, B=B, k=None, k_lo=k_lo, k_hi=k_hi, ctx_lo=ctx_lo, ctx_hi=ctx_hi, Hq=Hq,
                                Hkv=Hkv, D=D, H=H, V=V, max_pages=max_pages, w_std=1 / math.sqrt(H))


ATTN_CASES = [
    # name, B, k range, ctx range, Hq, Hkv, D, max_pages
    _wl("a64", 3, 0, 5, 1, 700, 4, 1, 64, 64),
    _wl("a128", 5, 1, 6, 200, 1100, 8, 2, 128, 80),
    _wl("a256", 2, 2, 6, 500, 900, 4, 1, 256, 64),
    _wl("agqa", 4, 3, 4, 50, 600, 32, 8, 128, 48),
    _wl("awide", 2, 6, 6, 100, 300, 16, 2, 256, 32),     # G*T = 56 rows per kv head
    _wl("atall", 2, 7, 7, 100, 300, 64, 4, 64, 32),      # G*T = 128 rows: both row groups
    _wl("adeep", 2, 30, 40, 100, 600, 32, 4, 128, 48),   # G*T up to 328 rows: six row groups
]


@pytest.mark.parametrize("split", [0, 64, 1024])   # 1024: pool read with non-temporal loads
def test_tiny_workload_attention(dev, split):
    x = synth.make_verify_inputs("tiny", seed=0)
    out, kp, vp, st = gpu_attn(x, dev, kv_split_tokens=split)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn(x)
    assert (st == 0).all() and (st_ref == 0).all()
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, "tiny attention")


@pytest.mark.parametrize("wl", ATTN_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1])
def test_attention_cases(dev, wl, seed):
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    print(f"[attn] {wl.name} seed {seed} pos {x.pos.tolist()} k {x.k.tolist()}", flush=True)
    out, kp, vp, st = gpu_attn(x, dev)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn(x)
    assert list(st) == list(st_ref) == [0] * len(x.pos)
    assert np.array_equal(bits(kp), kp_ref), "K pool differs from the oracle's append"
    assert np.array_equal(bits(vp), vp_ref), "V pool differs from the oracle's append"
    assert_close(out.float().cpu().numpy(), ref, f"attention {wl.name}")


def test_attention_rows_equal_one_row_decode(dev):
    """Row invariance: row j of a T-row verify is byte-identical to a one-row call at
    pos + j made after rows < j were appended (kv_hi = position)."""
    wl = _wl("inv", 3, 3, 6, 300, 1500, 8, 2, 128, 128)
    x = synth.make_verify_inputs(wl, seed=3, with_lm_head=False)
    out, _, _, st = gpu_attn(x, dev)
    assert (st == 0).all()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    kp, vp = x.k_pool.clone(), x.v_pool.clone()
    for s in range(len(x.pos)):
        for j in range(x.k[s] + 1):
            r = off[s] + j
            o1, kp, vp, st1 = gpu_attn(x, dev, pos=x.pos[s:s + 1] + j, k=np.zeros(1, np.int32),
                                       page_table=x.page_table[s:s + 1], k_pool=kp, v_pool=vp,
                                       q=x.q[r:r + 1], k_new=x.k_new[r:r + 1], v_new=x.v_new[r:r + 1])
            assert st1[0] == 0
            assert torch.equal(o1[0].view(torch.int16), out[r].view(torch.int16)), f"row {r} (seq {s}, j {j})"


@pytest.mark.parametrize("D", [64, 128, 256])
def test_attention_kmax_does_not_change_results(dev, D):
    """kmax only sizes the launch (one to eight 64-row groups): results are byte-identical."""
    wl = _wl(f"both{D}", 4, 0, 3, 10, 1500, 4, 1, D, 128)
    x = synth.make_verify_inputs(wl, seed=9, with_lm_head=False)
    small, _, _, st1 = gpu_attn(x, dev, kmax=3)       # 16 rows per kv head: one row group
    large, _, _, st2 = gpu_attn(x, dev, kmax=31)      # 128 rows: two row groups
    huge, _, _, st3 = gpu_attn(x, dev, kmax=127)      # 512 rows: eight row groups
    assert (st1 == 0).all() and (st2 == 0).all() and (st3 == 0).all()
    assert torch.equal(small.view(torch.int16), large.view(torch.int16))
    assert torch.equal(small.view(torch.int16), huge.view(torch.int16))
    _, ref, *_ = oracle_attn(x)
    assert_close(small.float().cpu().numpy(), ref, "both kernels")


def test_attention_split_sizes_agree(dev):
    wl = _wl("spl", 3, 2, 5, 1000, 2000, 8, 2, 128, 160)
    x = synth.make_verify_inputs(wl, seed=4, with_lm_head=False)
    outs = [gpu_attn(x, dev, kv_split_tokens=s)[0].float().cpu().numpy() for s in (64, 256, 1024)]
    _, ref, *_ = oracle_attn(x)
    for o in outs:
        assert_close(o, ref, "split")


def test_attention_error_paths(dev):
    wl = _wl("err", 4, 1, 3, 40, 200, 8, 2, 64, 32)
    x = synth.make_verify_inputs(wl, seed=5, with_lm_head=False)
    pt = x.page_table.copy()
    pt[1, 2] = x.n_pages + 3                 # page id out of range
    pos = x.pos.copy()
    pos[2] = 32 * 16 - 1                     # (pos + k) / 16 beyond the table
    out, kp, vp, st = gpu_attn(x, dev, page_table=pt, pos=pos)
    assert st[1] == synth_status("BAD_PAGE") and st[2] == synth_status("BAD_POS")
    assert st[0] == 0 and st[3] == 0
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    o = out.float().cpu().numpy()
    assert np.isnan(o[off[1]:off[3]]).all(), "flagged sequences must leave their rows untouched"
    # valid sequences are unaffected
    keep = [0, 3]
    rows, ref, *_ = oracle_attn(x, seqs=keep)
    assert_close(o[rows], ref, "valid rows next to flagged ones")
    # the flagged sequences wrote nothing into the pool
    ref_all_k, ref_all_v = oracle_attn(x, seqs=keep)[2:4]
    assert np.array_equal(bits(kp), ref_all_k) and np.array_equal(bits(vp), ref_all_v)
    # rows that do not add up: every sequence flagged
    out, _, _, st = gpu_attn(x, dev, k=x.k + np.array([0, 0, 0, 1], np.int32))
    assert (st == synth_status("BAD_ROWS")).all()
    assert np.isnan(out.float().cpu().numpy()).all()


def test_attention_rows_beyond_kmax(dev):
    """kmax bounds the launch: a sequence with k_s > kmax is flagged BAD_ROWS (and untouched);
    a kmax whose query rows exceed 128 per kv head is refused on the host."""
    import greedy_draft_verify_amd as gdv
    wl = _wl("wide", 3, 2, 5, 100, 200, 16, 1, 64, 32)
    x = synth.make_verify_inputs(wl, seed=6, with_lm_head=False)
    kmax = int(x.k.max()) - 1
    out, _, _, st = gpu_attn(x, dev, kmax=kmax)
    over = x.k > kmax
    assert over.any()
    assert (st[over] == synth_status("BAD_ROWS")).all() and (st[~over] == 0).all()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    o = out.float().cpu().numpy()
    for s in np.nonzero(over)[0]:
        assert np.isnan(o[off[s]:off[s + 1]]).all()
    with pytest.raises(gdv.SpecError):
        gpu_attn(x, dev, kmax=128)    # past the 127-draft limit


def synth_status(name):
    import greedy_draft_verify_amd as gdv
    return getattr(gdv, "STATUS_" + name)


# ---------------------------------------------------------------------------
# lm_head + argmax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R,H,V", [(1, 256, 1), (4, 256, 1024), (5, 256, 1000), (17, 768, 4097),
                                   (80, 512, 3000), (96, 256, 129), (130, 256, 777), (300, 256, 2000),
                                   (129, 256, 129), (200, 256, 100), (256, 512, 4097),
                                   (112, 512, 1000), (120, 256, 3000)])
def test_lm_head_shapes(dev, R, H, V):
    rng = np.random.default_rng(R * 1000 + V)
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    g, mv = gpu_lm_head(h, w, dev)
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(h), bits(w), R, H, V)
    n_undecided = check_argmax(g, mv, g_ref, t1, t2, f"lm_head R={R} H={H} V={V}")
    assert n_undecided <= max(2, R // 3)


def test_lm_head_pack_is_the_documented_permutation(dev):
    """Packed fragment (g, b, t, s, lane) holds w[128g + 16t + lane % 16][128b + 32s + 8(lane // 16) .. +8],
    zero past V (groups of 128 rows, K-blocks of 128 channels)."""
    import greedy_draft_verify_amd as gdv
    rng = np.random.default_rng(21)
    V, H = 150, 512
    w = torch.from_numpy(rng.standard_normal((V, H)).astype(np.float32)).to(torch.bfloat16)
    wp = bits(gdv.spec_lm_head_pack(w.to(dev)))
    torch.cuda.synchronize()
    wb = bits(w)
    ng, nb = (V + 127) // 128, H // 128
    exp = np.zeros((ng, nb, 8, 4, 64, 8), np.uint16)
    for g in range(ng):
        for b in range(nb):
            for t in range(8):
                for s in range(4):
                    for lane in range(64):
                        v = 128 * g + 16 * t + lane % 16
                        k = 128 * b + 32 * s + 8 * (lane // 16)
                        if v < V:
                            exp[g, b, t, s, lane] = wb[v, k:k + 8]
    assert wp.size == exp.size
    assert np.array_equal(wp.reshape(exp.shape), exp)


def test_lm_head_workspace_reuse(dev):
    """One zero-filled workspace serves consecutive calls of different sizes; every call
    leaves it zero and gives the same bytes as a call with a fresh workspace."""
    import greedy_draft_verify_amd as gdv
    rng = np.random.default_rng(31)
    H, V = 512, 2000
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    ws = gdv.workspace(gdv.lm_head_argmax_workspace_bytes(300, H, V), dev, zero=True)
    for R in (300, 7, 160, 300, 1):
        h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16).to(dev)
        am, mv = torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.float32, device=dev)
        gdv.spec_lm_head_argmax(h, wp, V, am, mv, workspace_buf=ws)
        am2, mv2 = torch.empty_like(am), torch.empty_like(mv)
        gdv.spec_lm_head_argmax(h, wp, V, am2, mv2)
        torch.cuda.synchronize()
        assert torch.equal(am, am2) and torch.equal(mv.view(torch.int32), mv2.view(torch.int32)), R
        assert int(ws.count_nonzero()) == 0, f"workspace not left zero after R={R}"


@pytest.mark.parametrize("R", [1, 5, 16, 33, 48, 64])
def test_lm_head_key_rows_path_equals_the_atomic_path(dev, R):
    """At R <= 64 the per-row maxima are merged by a second kernel from per-workgroup
    key rows; a workspace holding only the ticket and per-row keys makes the call merge
    them through the atomic keys instead. Both give the same bytes, and both leave the
    workspace zero."""
    import greedy_draft_verify_amd as gdv
    rng = np.random.default_rng(60 + R)
    H, V = 512, 20000
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16).to(dev)
    full = gdv.lm_head_argmax_workspace_bytes(R, H, V)
    small = 256 + 8 * R
    assert full > small
    outs = []
    for nbytes in (full, small):
        ws = gdv.workspace(nbytes, dev, zero=True)
        am, mv = torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.float32, device=dev)
        gdv.spec_lm_head_argmax(h, wp, V, am, mv, workspace_buf=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, nbytes
        outs.append((am.cpu(), mv.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(h), bits(w), R, H, V)
    check_argmax(outs[0][0].numpy(), outs[0][1].numpy(), g_ref, t1, t2, f"key rows R={R}")


def test_lm_head_tiny_workload(dev):
    x = synth.make_verify_inputs("tiny", seed=0)
    g, mv = gpu_lm_head(x.hidden, x.w, dev)
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(x.hidden), bits(x.w), x.R, x.wl.H, x.wl.V)
    check_argmax(g, mv, g_ref, t1, t2, "tiny lm_head")


def test_lm_head_rows_are_batch_invariant(dev):
    """A row's argmax and max logit are the same bytes whether it is scored alone or
    with 79 or 299 other rows (row groups of 128 included)."""
    rng = np.random.default_rng(7)
    H, V = 512, 5000
    import greedy_draft_verify_amd as gdv
    h = torch.from_numpy(rng.standard_normal((300, H)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    g300, m300 = gpu_lm_head(h, w, dev, wp)
    g80, m80 = gpu_lm_head(h[:80], w, dev, wp)
    assert np.array_equal(g80, g300[:80]) and np.array_equal(m80.view(np.uint32), m300[:80].view(np.uint32))
    for r in (0, 5, 79, 130, 299):
        g1, m1 = gpu_lm_head(h[r:r + 1], w, dev, wp)
        assert g1[0] == g300[r] and m1.view(np.uint32)[0] == m300.view(np.uint32)[r], r


def test_lm_head_ties_and_planted_winner(dev):
    rng = np.random.default_rng(8)
    R, H, V = 6, 256, 700
    hf = rng.standard_normal((R, H)).astype(np.float32)
    wf = (rng.standard_normal((V, H)) / 16).astype(np.float32)
    wf[513] = 3 * hf[0] / np.linalg.norm(hf[0])           # planted winner for row 0
    wf[77] = 3 * hf[1] / np.linalg.norm(hf[1])            # exact tie for row 1: 77 and 650
    wf[650] = wf[77]
    wf[699] = 3 * hf[2] / np.linalg.norm(hf[2])           # winner in the ragged last tile
    h = torch.from_numpy(hf).to(torch.bfloat16)
    w = torch.from_numpy(wf).to(torch.bfloat16)
    g, mv = gpu_lm_head(h, w, dev)
    assert g[0] == 513 and g[1] == 77 and g[2] == 699


# ---------------------------------------------------------------------------
# greedy accept
# ---------------------------------------------------------------------------
def test_accept_golden_cases(dev):
    from tests.test_oracle_pins import _load_accept_cases
    for name, g, drafts, d2t, a, emit, dpos in _load_accept_cases():
        k = len(drafts)
        kmax = max(k, 1)
        dr = np.full((1, kmax), -1, np.int32)
        dr[0, :k] = drafts
        res = gpu_accept(np.array(g), dr, np.array([k]), None if d2t is None else np.array(d2t), 1000,
                         np.array([100]), dev)
        assert res["status"][0] == 0, name
        assert res["accept_len"][0] == a and res["n_emit"][0] == len(emit), name
        assert list(res["emit"][0, :len(emit)]) == emit and (res["emit"][0, len(emit):] == -1).all(), name
        assert res["pos_out"][0] == 100 + dpos and res["next_tok"][0] == emit[-1], name


@pytest.mark.parametrize("B,kmax,use_d2t", [(1, 3, False), (16, 4, False), (64, 6, False), (8, 6, True),
                                            (300, 9, True), (5, 70, False), (2000, 3, False),
                                            (8192, 2, False), (3, 1024, True)])
def test_accept_random_vs_oracle(dev, B, kmax, use_d2t):
    rng = np.random.default_rng(B * 7 + kmax)
    V = 5000
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    d2t = rng.permutation(V)[:1000].astype(np.int32) if use_d2t else None
    inv = {int(t): i for i, t in enumerate(d2t)} if use_d2t else None
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.full((B, kmax), -1, np.int32)
    for s in range(B):
        for j in range(k[s]):
            t = g[off[s] + j]
            if rng.uniform() < 0.75:
                drafts[s, j] = inv.get(int(t), 0) if use_d2t else t
            else:
                drafts[s, j] = rng.integers(0, 1000 if use_d2t else V)
    pos = rng.integers(0, 100000, B).astype(np.int32)
    got = gpu_accept(g, drafts, k, d2t, V, pos, dev)
    ref = oracle.greedy_accept(g, drafts, kmax, k, d2t, 0 if d2t is None else len(d2t), V, B, R, pos)
    assert_accept_equal(got, ref, f"accept B={B}")


def test_accept_error_paths_vs_oracle(dev):
    V = 100
    k = np.array([2, 3, 1, 0], np.int32)
    R = int((k + 1).sum())
    g = np.arange(R, dtype=np.int32) % V
    drafts = np.array([[0, 1, 0], [3, 999, 5], [6, 0, 0], [0, 0, 0]], np.int32)   # seq 1 has an id >= V
    pos = np.array([5, 6, -1, 8], np.int32)                                          # seq 2 has pos < 0
    got = gpu_accept(g, drafts, k, None, V, pos, dev)
    ref = oracle.greedy_accept(g, drafts, 3, k, None, 0, V, 4, R, pos)
    assert_accept_equal(got, ref, "errors")
    assert list(ref["status"]) == [0, 8, 2, 0]
    # k beyond kmax, and rows that do not add up
    got = gpu_accept(g, drafts[:, :2], np.array([2, 3, 1, 0], np.int32), None, V, np.abs(pos), dev)
    ref = oracle.greedy_accept(g, drafts[:, :2], 2, np.array([2, 3, 1, 0], np.int32), None, 0, V, 4, R, np.abs(pos))
    assert_accept_equal(got, ref, "k > kmax")
    g2 = np.zeros(R + 1, np.int32)
    got = gpu_accept(g2, drafts, k, None, V, np.abs(pos), dev)
    ref = oracle.greedy_accept(g2, drafts, 3, k, None, 0, V, 4, R + 1, np.abs(pos))
    assert_accept_equal(got, ref, "rows mismatch")
    assert (ref["status"] == 4).all()
    # d2t entry out of range
    d2t = np.array([1, 2, 500], np.int32)
    got = gpu_accept(g, np.array([[0, 2, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0]], np.int32), k, d2t, V,
                     np.abs(pos), dev)
    ref = oracle.greedy_accept(g, np.array([[0, 2, 0], [0, 0, 0], [0, 0, 0], [0, 0, 0]], np.int32), 3, k, d2t, 3,
                               V, 4, R, np.abs(pos))
    assert_accept_equal(got, ref, "d2t range")
    assert ref["status"][0] == 8


def test_accept_in_place_positions(dev):
    import greedy_draft_verify_amd as gdv
    g = np.array([4, 5, 6, 7, 8], np.int32)
    drafts = np.array([[4, 9], [1, 1]], np.int32)
    k = np.array([2, 1], np.int32)
    pos = i32([10, 20], dev)
    z = lambda: torch.zeros(2, dtype=torch.int32, device=dev)
    acc, ne, nt, st = z(), z(), z(), z()
    emit = torch.zeros((2, 3), dtype=torch.int32, device=dev)
    gdv.spec_greedy_accept(i32(g, dev), i32(drafts, dev), i32(k, dev), None, 100, pos, pos, acc, ne, emit, nt, st)
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [12, 21] and acc.cpu().tolist() == [1, 0]
    assert emit.cpu().tolist() == [[4, 5, -1], [7, -1, -1]]


# ---------------------------------------------------------------------------
# Gated DeltaNet
# ---------------------------------------------------------------------------
def _delta_gpu(d, dev, mode, L=None, state=None):
    import greedy_draft_verify_amd as gdv
    st = (d.state if state is None else state).to(dev).clone()
    rec = torch.full((d.B, d.T, d.Hd, d.dv, d.dk), float("nan"), dtype=torch.float32, device=dev)
    o = torch.full((d.B, d.T, d.Hd, d.dv), float("nan"), dtype=torch.bfloat16, device=dev)
    gdv.spec_delta_verify_rollback(mode, d.q.to(dev), d.k.to(dev), d.v.to(dev), d.a.to(dev), d.b.to(dev), 1.0,
                                   st, rec, None if L is None else i32(L, dev), o)
    torch.cuda.synchronize()
    return st, rec, o


@pytest.mark.parametrize("B,T,Hd", [(1, 1, 1), (2, 5, 3), (3, 7, 2), (2, 37, 2), (1, 64, 1)])
def test_delta_record_vs_oracle(dev, B, T, Hd):
    d = synth.make_delta_inputs(seed=B + T, B=B, T=T, Hd=Hd)
    st, rec, o = _delta_gpu(d, dev, 1)
    rec_ref, o_ref = oracle.delta_verify(bits(d.q), bits(d.k), bits(d.v), d.a.numpy(), d.b.numpy(), 1.0,
                                         d.state.numpy(), B, T, Hd, 128, 128)
    assert_close(rec.cpu().numpy(), rec_ref, "delta record")
    assert_close(o.float().cpu().numpy(), o_ref, "delta output")
    assert torch.equal(st.cpu(), d.state), "mode 1 must not modify the state"


def test_delta_rollback_modes(dev):
    d = synth.make_delta_inputs(seed=11, B=6, T=5, Hd=2)
    L = np.array([0, 1, 2, 3, 5, 9], np.int32)          # 9 is clamped to T
    st3, rec3, o3 = _delta_gpu(d, dev, 3, L=L)
    st1, rec1, o1 = _delta_gpu(d, dev, 1)
    assert torch.equal(rec3, rec1) and torch.equal(o3.view(torch.int16), o1.view(torch.int16))
    import greedy_draft_verify_amd as gdv
    st2 = d.state.to(dev).clone()
    gdv.spec_delta_verify_rollback(2, None, None, None, None, None, 1.0, st2, rec1, i32(L, dev))
    torch.cuda.synchronize()
    assert torch.equal(st2, st3)
    for s in range(d.B):
        Ls = min(int(L[s]), d.T)
        want = d.state[s] if Ls == 0 else rec1[s, Ls - 1].cpu()
        assert torch.equal(st3[s].cpu(), want), s


def test_delta_input_stash_modes(dev):
    """VERIFY writes the record path's outputs and nothing else; RESCAN re-runs the
    committed prefix from the retained S_0 and leaves exactly the bytes ROLLBACK
    restores from the record (L = 0 keeps S_0, out-of-range L is clamped)."""
    import greedy_draft_verify_amd as gdv
    d = synth.make_delta_inputs(seed=14, B=7, T=19, Hd=2)
    L = np.array([0, 1, 5, 16, 17, 19, 40], np.int32)
    st1, rec1, o1 = _delta_gpu(d, dev, gdv.DELTA_RECORD)
    st2 = d.state.to(dev).clone()
    gdv.spec_delta_verify_rollback(gdv.DELTA_ROLLBACK, None, None, None, None, None, 1.0, st2, rec1, i32(L, dev))
    to = lambda t: t.to(dev)
    s4 = d.state.to(dev).clone()
    o4 = torch.full_like(o1, float("nan"))
    gdv.spec_delta_verify_rollback(gdv.DELTA_VERIFY, to(d.q), to(d.k), to(d.v), to(d.a), to(d.b), 1.0, s4, None,
                                   None, o4)
    s5 = d.state.to(dev).clone()
    gdv.spec_delta_verify_rollback(gdv.DELTA_RESCAN, to(d.q), to(d.k), to(d.v), to(d.a), to(d.b), 1.0, s5, None,
                                   i32(L, dev), None)
    torch.cuda.synchronize()
    assert torch.equal(o4.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(s4.cpu(), d.state), "VERIFY must not modify the state"
    assert torch.equal(s5, st2), "RESCAN must give the restored record's bytes"
    rec_ref, _ = oracle.delta_verify(bits(d.q), bits(d.k), bits(d.v), d.a.numpy(), d.b.numpy(), 1.0,
                                     d.state.numpy(), d.B, d.T, d.Hd, 128, 128)
    for s in range(d.B):
        Ls = min(int(L[s]), d.T)
        want = d.state[s].numpy() if Ls == 0 else rec_ref[s, Ls - 1]
        assert_close(s5[s].cpu().numpy(), want, f"RESCAN state, sequence {s}")


@pytest.mark.parametrize("T,Ls", [(5, (1, 2, 3, 4)), (20, (1, 15, 16, 17))])
def test_delta_record_is_prefix_invariant(dev, T, Ls):
    """S_L of a T-token scan equals the last state of an L-token scan, bit for bit (also
    across the 16-token rounds in which the scan stages its inputs)."""
    d = synth.make_delta_inputs(seed=12, B=2, T=T, Hd=2)
    _, rec, o = _delta_gpu(d, dev, 1)
    for L in Ls:
        e = synth.DeltaInputs(d.B, L, d.Hd, d.dk, d.dv, d.q[:, :L].contiguous(), d.k[:, :L].contiguous(),
                              d.v[:, :L].contiguous(), d.a[:, :L].contiguous(), d.b[:, :L].contiguous(), d.state, d.L)
        _, rl, ol = _delta_gpu(e, dev, 1)
        assert torch.equal(rl, rec[:, :L]) and torch.equal(ol.view(torch.int16), o[:, :L].view(torch.int16))


def test_delta_pure_decay(dev):
    d = synth.make_delta_inputs(seed=13, B=2, T=4, Hd=2)
    d.b.zero_()
    _, rec, _ = _delta_gpu(d, dev, 1)
    cum = torch.cumprod(d.a.double(), dim=1)
    for t in range(d.T):
        ref = (cum[:, t, :, None, None] * d.state.double()).numpy()
        assert_close(rec[:, t].cpu().numpy(), ref, "decay", atol=1e-5, rtol=1e-5)
