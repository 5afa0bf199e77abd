"""GPU parity of speculative sampling with dense draft distributions (DSSD fast.py
_sample_verify with the draft head's whole q) against the CPU oracle.

Bars:
  * z within |err| <= (2e-2 + 1e-2 |logit|) / T of the oracle's logit / T, lse within
    2e-2 + 1e-2 |lse|, and the draw from p equal wherever the oracle's winner beats its
    runner-up by more than 5e-2; the dense pass's lse and draw from p are the bytes of
    the support-list pass with no support;
  * the walk on identical per-row inputs (synthetic z, the oracle's lse and draws from
    p): outputs bit-exact for every sequence whose acceptance tests are decided
    beyond fp32 rounding (|log u - log(p/q)| > 1e-4) and whose deciding draw stays
    decided when p is known only to a relative 1e-5 (the oracle's robust gap: where
    p and q nearly cancel, log(p - q) is ill-conditioned);
  * end to end from the lm_head: outputs equal wherever the walk is decided by more
    than 5e-2 and the draw stays decided at a relative 5e-2 in p (the logits'
    tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import bits, i32

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

KEYS = ("status", "accept_len", "n_emit", "emit", "next_tok", "pos_out")


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def gpu_accept_dense(drafts, k, d2t, q, z, lse, sample_p, row_ctr, seed, pos, dev):
    import greedy_draft_verify_amd as gdv
    B, kmax = drafts.shape
    mk = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = mk(), mk(), mk(), mk(), mk()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    ws = gdv.workspace(gdv.sample_accept_dense_workspace_bytes(B), dev)
    ws.fill_(0xA5)                       # any contents: the call initialises what it uses
    gdv.spec_sample_accept_dense(i32(drafts, dev), i32(k, dev), None if d2t is None else i32(d2t, dev),
                                 q if torch.is_tensor(q) else _f32(q, dev), z if torch.is_tensor(z) else _f32(z, dev),
                                 _f32(lse, dev), i32(sample_p, dev), i32(row_ctr, dev), seed, i32(pos, dev), pos_out,
                                 acc, ne, emit, nt, st, workspace_buf=ws)
    torch.cuda.synchronize()
    return dict(status=st.cpu().numpy(), accept_len=acc.cpu().numpy(), n_emit=ne.cpu().numpy(),
                emit=emit.cpu().numpy(), next_tok=nt.cpu().numpy(), pos_out=pos_out.cpu().numpy())


def _dense_case(seed, B, kmax, V, sharp=2.0, closeness=0.5):
    """Target z per row, a draft distribution q near softmax(z) (how near: closeness),
    drafts drawn from q."""
    rng = np.random.default_rng(seed)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    z = rng.normal(0, sharp, (R, V)).astype(np.float32)
    zq = closeness * z + (1 - closeness) * rng.normal(0, sharp, (R, V))
    q = np.exp(zq - zq.max(1, keepdims=True))
    q = (q / q.sum(1, keepdims=True)).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.zeros((B, max(kmax, 1)), np.int32)[:, :kmax]
    for s in range(B):
        for j in range(k[s]):
            pr = q[off[s] + j].astype(np.float64)
            drafts[s, j] = rng.choice(V, p=pr / pr.sum())
    row_ctr = np.stack([rng.integers(0, 1 << 20, R), rng.integers(0, 1 << 30, R)], 1).astype(np.int32)
    pos = rng.integers(0, 5000, B).astype(np.int32)
    return k, R, z, q, drafts, row_ctr, pos


@pytest.mark.parametrize("B,kmax,V,closeness", [(64, 6, 5000, 0.9), (16, 4, 151936, 0.7), (200, 3, 1000, 0.0),
                                                (8, 0, 3000, 0.5)])
def test_dense_walk_parity_on_identical_rows(dev, B, kmax, V, closeness):
    print(f"dense walk B={B} kmax={kmax} V={V} closeness={closeness}", flush=True)
    seed = 0xfeed_0000_0000_0001 + V
    k, R, z, q, drafts, row_ctr, pos = _dense_case(B + V, B, kmax, V, closeness=closeness)
    logits = z.astype(np.float64)                      # T = 1: z is the logit
    rows = oracle.sample_rows(logits, 1.0, np.zeros((R, 0), np.int32), np.zeros((R, 0), np.float32), row_ctr, seed)
    ref = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, logits, 1.0, q, row_ctr, seed, pos, rel=1e-5)
    got = gpu_accept_dense(drafts, k, None, q, z, rows["lse"], rows["sample_p"], row_ctr, seed, pos, dev)
    decided = (ref["margin"] > 1e-4) & (ref["gap"] > 1e-4)
    assert decided.mean() > 0.9, decided.mean()
    for key in KEYS:
        assert np.array_equal(got[key][decided], ref[key][decided]), (key, got[key][decided][:5], ref[key][decided][:5])
    assert (ref["status"] == 0).all()
    if kmax:
        assert 0 < ref["accept_len"].sum() < k.sum() or closeness == 0.0


def test_dense_walk_error_paths(dev):
    B, kmax, V = 6, 3, 700
    rng = np.random.default_rng(9)
    k = np.array([3, 2, 3, 1, 0, 3], np.int32)
    R = int((k + 1).sum())
    z = rng.normal(0, 2.0, (R, V)).astype(np.float32)
    q = rng.uniform(0.5, 1.5, (R, V))
    q = (q / q.sum(1, keepdims=True)).astype(np.float32)
    drafts = rng.integers(0, V, (B, kmax)).astype(np.int32)
    row_ctr = np.stack([np.arange(R), np.full(R, 9)], 1).astype(np.int32)
    pos = rng.integers(0, 500, B).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    q[off[0] + 1, drafts[0, 1]] = 0.0          # a draft the draft distribution cannot produce
    drafts[2, 2] = V + 3                        # outside the vocabulary
    pos[3] = -1
    rows = oracle.sample_rows(z.astype(np.float64), 1.0, np.zeros((R, 0), np.int32), np.zeros((R, 0), np.float32),
                              row_ctr, 5)
    ref = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, z.astype(np.float64), 1.0, q, row_ctr, 5, pos)
    got = gpu_accept_dense(drafts, k, None, q, z, rows["lse"], rows["sample_p"], row_ctr, 5, pos, dev)
    assert ref["status"][0] == oracle.BAD_TOKEN and ref["status"][2] == oracle.BAD_TOKEN
    assert ref["status"][3] == oracle.BAD_POS
    assert np.array_equal(got["status"], ref["status"])
    flagged = ref["status"] != 0
    for key in KEYS:
        assert np.array_equal(got[key][flagged], ref[key][flagged]), key
    # undefined packing (k_0 > kmax and the rows do not add up) flags every sequence
    k_bad = k.copy()
    k_bad[0] += 1
    bad = gpu_accept_dense(drafts, k_bad, None, q, z, rows["lse"], rows["sample_p"], row_ctr, 5, np.abs(pos), dev)
    assert (bad["status"] & oracle.BAD_ROWS).all() and (bad["emit"] == -1).all()
    assert (bad["pos_out"] == np.abs(pos)).all() and (bad["accept_len"] == -1).all()


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_dense_end_to_end_from_the_lm_head(dev, T):
    """lm_head pass with z kept, then the walk, against the oracle's fp64 logits; the
    pass's lse and draw from p equal the support-list pass with no support. Sequences
    the fp64 logits leave undecided (within the logits' tolerance) are compared with the
    oracle's walk over the GPU's own z, decided beyond fp32 rounding, so that nearly
    every sequence is compared one way or the other."""
    import greedy_draft_verify_amd as gdv
    B, kmax, V, H = 32, 4, 4096, 256
    rng = np.random.default_rng(17)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = torch.Generator().manual_seed(21)
    hidden = torch.randn((R, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, H), generator=g) / 8).to(torch.bfloat16)
    logits = oracle.lm_head_logits(bits(hidden), bits(w), R, H, V)
    # q near the target distribution, drafts drawn from q
    zq = 0.8 * logits / T + 0.2 * rng.normal(0, 2.0, (R, V))
    q = np.exp(zq - zq.max(1, keepdims=True))
    q = (q / q.sum(1, keepdims=True)).astype(np.float32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.zeros((B, kmax), np.int32)
    for s in range(B):
        for j in range(k[s]):
            pr = q[off[s] + j].astype(np.float64)
            drafts[s, j] = rng.choice(V, p=pr / pr.sum())
    row_ctr = np.stack([np.arange(R) + 40, np.full(R, 3)], 1).astype(np.int32)
    pos = rng.integers(0, 900, B).astype(np.int32)
    seed = 0x5eed
    wp = gdv.spec_lm_head_pack(w.to(dev))
    lse = torch.zeros(R, device=dev)
    sp = torch.zeros(R, dtype=torch.int32, device=dev)
    zt = torch.zeros((R, V), device=dev)
    gdv.spec_lm_head_sample_dense(hidden.to(dev), wp, V, T, i32(row_ctr, dev), seed, lse, sp, zt)
    # the support-list pass with no support: same lse and draw
    lse2 = torch.zeros(R, device=dev)
    sp2 = torch.zeros(R, dtype=torch.int32, device=dev)
    sr2 = torch.zeros(R, dtype=torch.int32, device=dev)
    e0 = torch.zeros((R, 0), dtype=torch.int32, device=dev)
    gdv.spec_lm_head_sample(hidden.to(dev), wp, V, T, e0, e0.float(), i32(row_ctr, dev), seed, lse2,
                            torch.zeros((R, 0), device=dev), sp2, sr2)
    torch.cuda.synchronize()
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32)) and torch.equal(sp, sp2)
    zg = zt.cpu().numpy().astype(np.float64)
    ztol = (2e-2 + 1e-2 * np.abs(logits)) / T
    assert (np.abs(zg - logits / T) <= ztol).all(), np.abs(zg - logits / T).max()
    rows = oracle.sample_rows(logits, T, np.zeros((R, 0), np.int32), np.zeros((R, 0), np.float32), row_ctr, seed)
    lg = lse.cpu().numpy().astype(np.float64)
    assert (np.abs(lg - rows["lse"]) <= 2e-2 + 1e-2 * np.abs(rows["lse"])).all()
    dec = rows["gap_p"] > 5e-2
    assert np.array_equal(sp.cpu().numpy()[dec], rows["sample_p"][dec])
    ref = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, logits, T, q, row_ctr, seed, pos, rel=5e-2)
    got = gpu_accept_dense(drafts, k, None, q, zt, lse.cpu().numpy(), sp.cpu().numpy(), row_ctr, seed, pos, dev)
    decided = (ref["margin"] > 5e-2) & (ref["gap"] > 0)
    assert decided.mean() > 0.5, decided.mean()
    for key in KEYS:
        assert np.array_equal(got[key][decided], ref[key][decided]), key
    # the same walk over the GPU's z (as fp64 logits): decided beyond fp32 rounding
    ref_g = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, zg * T, T, q, row_ctr, seed, pos, rel=1e-5)
    tight = (ref_g["margin"] > 1e-4) & (ref_g["gap"] > 1e-4)
    for key in KEYS:
        assert np.array_equal(got[key][tight], ref_g[key][tight]), key
    covered = decided | tight
    print(f"T={T}: {int(decided.sum())} of {B} sequences decided on fp64 logits, {int(tight.sum())} on the GPU's z, "
          f"{int(covered.sum())} compared")
    assert tight.mean() > 0.9 and covered.mean() >= 0.9, (tight.mean(), covered.mean())


def test_dense_pass_b16k4_rows(dev):
    """The b16k4 lm_head (H = 4096, V = 151936, 80 rows) at temperature 0.1, as the
    benchmark runs it: every fifth row's z, lse and draw from p against the oracle."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16k4", seed=0, device=dev)
    R, H, V, T = x.R, x.wl.H, x.wl.V, 0.1
    row_ctr = np.stack([np.arange(R) + 900, np.arange(R) // 5], 1).astype(np.int32)
    wp = gdv.spec_lm_head_pack(x.w)
    lse = torch.zeros(R, device=dev)
    sp = torch.zeros(R, dtype=torch.int32, device=dev)
    z = torch.zeros((R, V), device=dev)
    gdv.spec_lm_head_sample_dense(x.hidden, wp, V, T, i32(row_ctr, dev), 41, lse, sp, z)
    torch.cuda.synchronize()
    rows = np.arange(0, R, 5)
    logits = oracle.lm_head_logits(bits(x.hidden)[rows], bits(x.w), len(rows), H, V)
    ref = oracle.sample_rows(logits, T, np.zeros((len(rows), 0), np.int32), np.zeros((len(rows), 0), np.float32),
                             row_ctr[rows], 41)
    zg = z.cpu().numpy()[rows].astype(np.float64)
    ztol = (2e-2 + 1e-2 * np.abs(logits)) / T
    assert (np.abs(zg - logits / T) <= ztol).all(), np.abs(zg - logits / T).max()
    lg = lse.cpu().numpy()[rows].astype(np.float64)
    assert (np.abs(lg - ref["lse"]) <= (2e-2 + 1e-2 * np.abs(ref["lse"])) / T).all()
    dec = ref["gap_p"] > 5e-2 / T
    assert dec.mean() > 0.5
    assert np.array_equal(sp.cpu().numpy()[rows][dec], ref["sample_p"][dec])


@pytest.mark.parametrize("R,V", [(37, 1001), (128, 1030), (200, 515), (1, 3)])
def test_dense_pass_ragged_shapes(dev, R, V):
    """z of every entry on ragged shapes: a vocabulary that is not a multiple of 4 (the
    element-wise tail of the row stores) nor of a workgroup's 128 entries, an odd
    number of 16-row tiles, 8 tiles, and two row groups; plus lse and the draw from p."""
    import greedy_draft_verify_amd as gdv
    H, T, seed = 256, 0.7, 77
    print(f"dense pass R={R} V={V}", flush=True)
    g = torch.Generator().manual_seed(R * 7 + V)
    hidden = torch.randn((R, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, H), generator=g) / 8).to(torch.bfloat16)
    row_ctr = np.stack([np.arange(R) + 3, np.full(R, 9)], 1).astype(np.int32)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    lse = torch.zeros(R, device=dev)
    sp = torch.zeros(R, dtype=torch.int32, device=dev)
    z = torch.full((R, V), float("nan"), device=dev)
    gdv.spec_lm_head_sample_dense(hidden.to(dev), wp, V, T, i32(row_ctr, dev), seed, lse, sp, z)
    torch.cuda.synchronize()
    logits = oracle.lm_head_logits(bits(hidden), bits(w), R, H, V)
    zg = z.cpu().numpy().astype(np.float64)
    ztol = (2e-2 + 1e-2 * np.abs(logits)) / T
    assert (np.abs(zg - logits / T) <= ztol).all(), np.nanmax(np.abs(zg - logits / T))
    ref = oracle.sample_rows(logits, T, np.zeros((R, 0), np.int32), np.zeros((R, 0), np.float32), row_ctr, seed)
    lg = lse.cpu().numpy().astype(np.float64)
    assert (np.abs(lg - ref["lse"]) <= (2e-2 + 1e-2 * np.abs(ref["lse"])) / T).all()
    dec = ref["gap_p"] > 5e-2 / T
    assert np.array_equal(sp.cpu().numpy()[dec], ref["sample_p"][dec])
