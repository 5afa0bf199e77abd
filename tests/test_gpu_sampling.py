"""GPU parity of speculative-sampling verify against the CPU oracle.

DSSD fast.py _sample_verify, oxinfer speculative_accept, memra's counter-based
Philox note. Bars:
  * lse and the support z's within |err| <= 2e-2 + 1e-2 |ref|;
  * each Gumbel-max draw equal to the oracle's wherever the oracle's winner beats
    its runner-up by more than 5e-2 (both sides draw the same noise from the same
    counters; only the logits' rounding differs, as for the greedy argmax);
  * the chain walk bit-exact on identical per-row inputs, except rows whose
    acceptance uniform lies within 1e-4 (relative) of p/q;
  * statistically, the emitted tokens follow the target distribution (the
    method's theorem), and the zero-temperature limit gives the greedy walk.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, bits, i32

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

GAP = 5e-2


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def gpu_sample_rows(hidden, w_packed, V, T, q_tok, q_prob, row_ctr, seed, dev, ws=None):
    import greedy_draft_verify_amd as gdv
    R = hidden.shape[0]
    NQ = q_tok.shape[1]
    lse = torch.full((R,), float("nan"), device=dev)
    z = torch.full((R, NQ), -7.0, device=dev)
    sp = torch.full((R,), -9, dtype=torch.int32, device=dev)
    sr = torch.full((R,), -9, dtype=torch.int32, device=dev)
    gdv.spec_lm_head_sample(hidden, w_packed, V, T, i32(q_tok, dev), _f32(q_prob, dev), i32(row_ctr, dev), seed, lse,
                            z, sp, sr, workspace_buf=ws)
    torch.cuda.synchronize()
    return dict(lse=lse.cpu().numpy(), z_supp=z.cpu().numpy(), sample_p=sp.cpu().numpy(),
                sample_res=sr.cpu().numpy())


def _support(rng, R, V, NQ, point_rows=()):
    """Random sparse supports: some unused entries, some duplicated tokens."""
    q_tok = np.full((R, NQ), -1, np.int32)
    q_prob = np.zeros((R, NQ), np.float32)
    for r in range(R):
        n = int(rng.integers(0, NQ + 1))
        toks = rng.integers(0, V, n)
        if n >= 2 and rng.uniform() < 0.3:
            toks[1] = toks[0]                       # a duplicate entry
        q_tok[r, :n] = toks
        w = rng.uniform(0.05, 1.0, n)
        q_prob[r, :n] = (w / w.sum()).astype(np.float32)
    return q_tok, q_prob


def _check_rows(got, ref, what, min_decided=0.8):
    assert_close(got["lse"], ref["lse"], f"{what} lse")
    nan_ref = np.isnan(ref["z_supp"])
    assert np.array_equal(np.isnan(got["z_supp"]), nan_ref), f"{what}: unused support entries"
    assert_close(got["z_supp"][~nan_ref], ref["z_supp"][~nan_ref], f"{what} z_supp")
    for key, gk in (("sample_p", "gap_p"), ("sample_res", "gap_res")):
        dec = ref[gk] > GAP
        bad = np.nonzero(dec & (got[key] != ref[key]))[0]
        assert len(bad) == 0, f"{what} {key}: rows {bad[:8]} gpu {got[key][bad[:8]]} ref {ref[key][bad[:8]]}"
        assert dec.mean() >= min_decided, f"{what} {key}: only {dec.mean():.2f} of rows decided"


@pytest.mark.parametrize("R,V,NQ,T", [(37, 1000, 4, 0.7), (80, 1000, 8, 1.0), (160, 4099, 1, 1.3),
                                      (300, 2048, 0, 1.0), (5, 130, 8, 0.5), (96, 2000, 3, 1.1),
                                      (128, 1000, 8, 0.9), (256, 1030, 2, 0.8)])
def test_lm_head_sample_parity(dev, R, V, NQ, T):
    import greedy_draft_verify_amd as gdv
    print(f"lm_head sample R={R} V={V} NQ={NQ} T={T}", flush=True)
    H = 256
    rng = np.random.default_rng(R * 31 + V)
    g = torch.Generator().manual_seed(R + V)
    hidden = torch.randn((R, H), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, H), generator=g) / 8).to(torch.bfloat16)
    q_tok, q_prob = _support(rng, R, V, NQ)
    row_ctr = np.stack([rng.integers(0, 1 << 20, R), rng.integers(0, 1 << 30, R)], 1).astype(np.int32)
    seed = 0x0123_4567_89ab_cdef
    wp = gdv.spec_lm_head_pack(w.to(dev))
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, H, V), dev, zero=True)
    got = gpu_sample_rows(hidden.to(dev), wp, V, T, q_tok, q_prob, row_ctr, seed, dev, ws=ws)
    logits = oracle.lm_head_logits(bits(hidden), bits(w), R, H, V)
    ref = oracle.sample_rows(logits, T, q_tok, q_prob, row_ctr, seed)
    _check_rows(got, ref, f"R={R} V={V}")
    # a second call with the same workspace gives the same bytes
    again = gpu_sample_rows(hidden.to(dev), wp, V, T, q_tok, q_prob, row_ctr, seed, dev, ws=ws)
    for key in ("lse", "sample_p", "sample_res"):
        assert np.array_equal(again[key], got[key]), key
    # row invariance: the first rows alone give the same bytes
    part = gpu_sample_rows(hidden[:3].to(dev), wp, V, T, q_tok[:3], q_prob[:3], row_ctr[:3], seed, dev)
    for key in ("lse", "sample_p", "sample_res"):
        assert np.array_equal(part[key], got[key][:3]), key


def test_lm_head_sample_b16k4_rows(dev):
    """The b16k4 lm_head (H = 4096, V = 151936, 80 rows) at temperature 1 with point-mass
    supports, 16 of the rows checked against the oracle."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16k4", seed=0, device=dev)
    R, H, V = x.R, x.wl.H, x.wl.V
    rng = np.random.default_rng(3)
    q_tok = rng.integers(0, V, (R, 1)).astype(np.int32)
    q_prob = np.ones((R, 1), np.float32)
    row_ctr = np.stack([np.arange(R) + 500, np.arange(R) // 5], 1).astype(np.int32)
    wp = gdv.spec_lm_head_pack(x.w)
    got = gpu_sample_rows(x.hidden, wp, V, 1.0, q_tok, q_prob, row_ctr, 77, dev)
    rows = np.arange(0, R, 5)
    logits = oracle.lm_head_logits(bits(x.hidden)[rows], bits(x.w), len(rows), H, V)
    ref = oracle.sample_rows(logits, 1.0, q_tok[rows], q_prob[rows], row_ctr[rows], 77)
    sub = {k: v[rows] for k, v in got.items()}
    _check_rows(sub, ref, "b16k4 rows", min_decided=0.5)


def _accept_case(rng, B, kmax, V, NQ, T=1.0):
    """Per-row inputs computed by the oracle (from random logits), drafts drawn from
    their q."""
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    off = np.concatenate([[0], np.cumsum(k + 1)])
    logits = rng.standard_normal((R, V)) * 2
    logits[np.arange(R), rng.integers(0, V, R)] += 7.0   # a clear favourite per row
    q_tok = np.full((R, NQ), -1, np.int32)
    q_prob = np.zeros((R, NQ), np.float32)
    drafts = np.full((B, max(kmax, 1)), -1, np.int32)[:, :kmax]
    for s in range(B):
        for j in range(k[s]):
            r = off[s] + j
            n = int(rng.integers(1, NQ + 1))
            # the support: n of the row's 2n most likely tokens, so that drafts are often kept
            top = np.argsort(logits[r])[::-1][:2 * n]
            toks = rng.choice(top, n, replace=False)
            if n > 1 and rng.uniform() < 0.3:
                toks[-1] = toks[0]                  # a token listed twice: its q is the summed mass
            w = rng.uniform(0.05, 1, n)
            q_tok[r, :n] = toks
            q_prob[r, :n] = (w / w.sum()).astype(np.float32)
            drafts[s, j] = toks[rng.choice(n, p=(w / w.sum()))]
    row_ctr = np.stack([np.arange(R) + 7, np.repeat(np.arange(B), k + 1)], 1).astype(np.int32)
    rows = oracle.sample_rows(logits, T, q_tok, q_prob, row_ctr, 5)
    pos = rng.integers(0, 4000, B).astype(np.int32)
    return dict(k=k, R=R, off=off, q_tok=q_tok, q_prob=q_prob, drafts=drafts, row_ctr=row_ctr, rows=rows, pos=pos,
                V=V, B=B, kmax=kmax)


def gpu_sample_accept(c, dev, seed=5, d2t=None):
    import greedy_draft_verify_amd as gdv
    B, kmax = c["B"], c["kmax"]
    z = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = z(), z(), z(), z(), z()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    rows = c["rows"]
    gdv.spec_sample_accept(i32(c["drafts"], dev), i32(c["k"], dev), None if d2t is None else i32(d2t, dev), c["V"],
                           i32(c["q_tok"], dev), _f32(c["q_prob"], dev), _f32(rows["lse"], dev),
                           _f32(rows["z_supp"], dev), i32(rows["sample_p"], dev), i32(rows["sample_res"], dev),
                           i32(c["row_ctr"], dev), seed, i32(c["pos"], dev), pos_out, acc, ne, emit, nt, st)
    torch.cuda.synchronize()
    return dict(pos_out=pos_out.cpu().numpy(), accept_len=acc.cpu().numpy(), n_emit=ne.cpu().numpy(),
                emit=emit.cpu().numpy(), next_tok=nt.cpu().numpy(), status=st.cpu().numpy())


def _undecided_seqs(c, seed=5):
    """Sequences with a draft row whose uniform is within 1e-4 (relative) of p/q."""
    out = set()
    for s in range(c["B"]):
        for j in range(c["k"][s]):
            r = c["off"][s] + j
            hold = np.nonzero(c["q_tok"][r] == c["drafts"][s, j])[0]
            q_x = float(c["q_prob"][r, hold].astype(np.float64).sum())
            ratio = math.exp(c["rows"]["z_supp"][r, hold[0]] - c["rows"]["lse"][r]) / q_x
            u = oracle.accept_uniform(c["row_ctr"][r], seed)
            if abs(u - ratio) <= 1e-4 * max(ratio, 1e-30):
                out.add(s)
    return out


@pytest.mark.parametrize("B,kmax,V,NQ", [(16, 4, 300, 1), (64, 6, 500, 8), (4096, 3, 200, 4), (8, 70, 100, 2)])
def test_sample_accept_parity(dev, B, kmax, V, NQ):
    print(f"sample accept B={B} kmax={kmax} NQ={NQ}", flush=True)
    rng = np.random.default_rng(B + kmax)
    c = _accept_case(rng, B, kmax, V, NQ)
    ref = oracle.sample_accept(c["drafts"], kmax, c["k"], None, 0, V, B, c["R"], c["q_tok"], c["q_prob"], c["rows"],
                               c["row_ctr"], 5, c["pos"])
    got = gpu_sample_accept(c, dev)
    skip = _undecided_seqs(c)
    keep = np.array([s not in skip for s in range(B)])
    assert keep.mean() > 0.99
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit"):
        assert np.array_equal(got[key][keep], ref[key][keep]), key
    assert (ref["status"] == 0).all()
    assert 0 < ref["accept_len"].mean()


def test_sample_accept_error_paths(dev):
    rng = np.random.default_rng(1)
    c = _accept_case(rng, 6, 3, 50, 2)
    c["k"] = np.array([3, 3, 3, 3, 3, 3], np.int32)
    c = _accept_case(np.random.default_rng(2), 6, 3, 50, 2)
    ks = c["k"]
    drafts = c["drafts"].copy()
    s_bad = int(np.nonzero(ks > 0)[0][0])
    drafts[s_bad, 0] = (c["q_tok"][c["off"][s_bad], 0] + 1) % 50    # maybe outside its support
    if drafts[s_bad, 0] in c["q_tok"][c["off"][s_bad]]:
        drafts[s_bad, 0] = 60                                         # outside the vocabulary
    pos = c["pos"].copy()
    pos[-1] = -3
    c2 = dict(c, drafts=drafts, pos=pos)
    ref = oracle.sample_accept(drafts, 3, ks, None, 0, 50, 6, c["R"], c["q_tok"], c["q_prob"], c["rows"],
                               c["row_ctr"], 5, pos)
    got = gpu_sample_accept(c2, dev)
    assert ref["status"][s_bad] == oracle.BAD_TOKEN and ref["status"][-1] & oracle.BAD_POS
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit"):
        assert np.array_equal(got[key], ref[key]), key


def test_gpu_sampling_emits_the_target_distribution(dev):
    """The method's theorem through the GPU pipeline (spec_lm_head_sample ->
    spec_sample_accept): 4096 sequences with one point-mass draft each and the same
    two hidden rows; the first emitted token follows p(row 0), the token after an
    accepted draft follows p(row 1), and a draft is kept with probability p(x)."""
    import greedy_draft_verify_amd as gdv
    B, V, H, T = 4096, 1000, 256, 0.8
    g = torch.Generator().manual_seed(4)
    w = (torch.randn((V, H), generator=g) / 6).to(torch.bfloat16)
    h2 = torch.randn((2, H), generator=g).to(torch.bfloat16)
    hidden = h2.repeat(B, 1).contiguous()
    R = 2 * B
    logits = oracle.lm_head_logits(bits(h2), bits(w), 2, H, V)
    p0 = np.exp(logits[0] / T - logits[0].max() / T)
    p0 /= p0.sum()
    p1 = np.exp(logits[1] / T - logits[1].max() / T)
    p1 /= p1.sum()
    x = int(np.argsort(p0)[-2])                          # the runner-up as the draft
    q_tok = np.full((R, 1), -1, np.int32)
    q_tok[0::2, 0] = x
    q_prob = np.zeros((R, 1), np.float32)
    q_prob[0::2, 0] = 1.0
    row_ctr = np.stack([np.tile([900, 901], B), np.repeat(np.arange(B), 2)], 1).astype(np.int32)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    rows = gpu_sample_rows(hidden.to(dev), wp, V, T, q_tok, q_prob, row_ctr, 2024, dev)
    c = dict(k=np.ones(B, np.int32), R=R, q_tok=q_tok, q_prob=q_prob, drafts=np.full((B, 1), x, np.int32),
             row_ctr=row_ctr, rows=rows, pos=np.full(B, 900, np.int32), V=V, B=B, kmax=1)
    res = gpu_sample_accept(c, dev, seed=2024)
    assert (res["status"] == 0).all()

    def band(tokens, p, what):
        n = len(tokens)
        top = np.argsort(p)[::-1][:6]
        for t in top:
            cnt = int((tokens == t).sum())
            sd = math.sqrt(n * p[t] * (1 - p[t]))
            assert abs(cnt - n * p[t]) <= 5 * sd + 1, (what, t, cnt, n * p[t])
        other = 1 - p[top].sum()
        cnt = int((~np.isin(tokens, top)).sum())
        assert abs(cnt - n * other) <= 5 * math.sqrt(n * other * (1 - other)) + 1, (what, "other", cnt, n * other)

    band(res["emit"][:, 0], p0, "first token")
    acc = res["accept_len"] == 1
    assert abs(acc.mean() - p0[x]) <= 5 * math.sqrt(p0[x] * (1 - p0[x]) / B)
    band(res["emit"][acc, 1], p1, "bonus after an accepted draft")
    assert (res["emit"][~acc, 0] != x).all()


def test_gpu_zero_temperature_is_greedy(dev):
    """Temperature 1e-3 with point-mass drafts: the sampled walk equals the greedy oracle
    wherever the greedy decisions are decided (top-2 logit gap > 5e-2)."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("tiny", seed=0, device=dev)
    H, V = x.wl.H, x.wl.V
    B, kmax = 32, 4
    rng = np.random.default_rng(6)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    hidden = synth.normal_bf16((R, H), 4.0, 3, "tiny", "extra", dev)   # logits of std ~4: clear greedy picks
    g, t1, t2, _ = oracle.lm_head_argmax(bits(hidden), bits(x.w), R, H, V)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.full((B, kmax), -1, np.int32)
    for s in range(B):
        for j in range(k[s]):
            drafts[s, j] = g[off[s] + j] if rng.uniform() < 0.7 else rng.integers(0, V)
    q_tok = np.full((R, 1), -1, np.int32)
    q_prob = np.zeros((R, 1), np.float32)
    for s in range(B):
        for j in range(k[s]):
            q_tok[off[s] + j, 0] = drafts[s, j]
            q_prob[off[s] + j, 0] = 1.0
    row_ctr = np.stack([np.arange(R), np.zeros(R)], 1).astype(np.int32)
    wp = gdv.spec_lm_head_pack(x.w)
    rows = gpu_sample_rows(hidden, wp, V, 1e-3, q_tok, q_prob, row_ctr, 11, dev)
    pos = rng.integers(0, 100, B).astype(np.int32)
    c = dict(k=k, R=R, q_tok=q_tok, q_prob=q_prob, drafts=drafts, row_ctr=row_ctr, rows=rows, pos=pos, V=V, B=B,
             kmax=kmax)
    got = gpu_sample_accept(c, dev, seed=11)
    ref = oracle.greedy_accept(g, drafts, kmax, k, None, 0, V, B, R, pos)
    decided = np.array([(t1 - t2)[off[s]:off[s + 1]].min() > GAP for s in range(B)])
    assert decided.mean() > 0.6
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit"):
        assert np.array_equal(got[key][decided], ref[key][decided]), key
