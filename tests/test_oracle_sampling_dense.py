"""Pins of the oracle's speculative sampling with a dense draft distribution, CPU only.

DSSD fast.py _sample_verify verifies drafts drawn from the draft head's full
distribution q: draft x is kept with probability min(1, p(x)/q(x)); at the first
rejection the token is drawn from norm(max(p - q, 0)); if every draft is kept the
bonus is drawn from p.

The pins:
  * the theorem the method rests on: the first emitted token is distributed as p
    whatever q is, the acceptance rate is sum_x min(p(x), q(x)), and after an
    accepted draft the next token is distributed as the next row's p (binomial
    5-sigma bands);
  * a dense q that vanishes outside a few tokens is the sparse case: the walk must
    give exactly the outputs of the support-list formulation (whose residual is
    formed differently: support entries get p - q, all others p);
  * error paths (zero-mass drafts, out-of-range ids, undefined packing, d2t).
"""
import numpy as np
import pytest

import oracle


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _band(counts, probs, n, sigmas=5.0):
    exp = probs * n
    sd = np.sqrt(n * probs * (1 - probs)) + 1e-9
    return np.all(np.abs(counts - exp) <= sigmas * sd + 1), (counts, exp)


def _one_draft_dense(B, p_logits, p2_logits, q, rng, T=1.0):
    V = len(p_logits)
    x = rng.choice(V, size=B, p=q)
    R = 2 * B
    logits = np.empty((R, V))
    logits[0::2] = p_logits
    logits[1::2] = p2_logits
    qd = np.zeros((R, V), np.float32)
    qd[0::2] = q
    row_ctr = np.stack([np.tile([100, 101], B), np.repeat(np.arange(B), 2)], 1).astype(np.int32)
    res = oracle.sample_accept_dense(x[:, None], 1, np.ones(B, np.int32), None, 0, V, B, R, logits, T, qd,
                                     row_ctr, 99, np.full(B, 100, np.int32))
    assert (res["status"] == 0).all()
    return x, res


@pytest.mark.parametrize("q", [np.array([0.1, 0.15, 0.3, 0.25, 0.2]),     # dense, unlike p
                               np.array([0.05, 0.4, 0.05, 0.3, 0.2]),     # dense, close to p
                               np.array([0.0, 0.0, 0.9, 0.1, 0.0])])      # zero entries
def test_dense_speculative_sampling_emits_the_target_distribution(q):
    rng = np.random.default_rng(7)
    B = 60000
    p_logits = np.array([0.3, 1.2, -0.4, 0.8, 0.0])
    p2_logits = np.array([-1.0, 0.0, 2.0, 0.5, 0.1])
    x, res = _one_draft_dense(B, p_logits, p2_logits, q, rng)
    p = _softmax(p_logits)
    ok, info = _band(np.bincount(res["emit"][:, 0], minlength=5), p, B)
    assert ok, info
    acc = res["accept_len"] == 1
    rate = np.minimum(p, q).sum()
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / B)
    ok, info = _band(np.bincount(res["emit"][acc, 1], minlength=5), _softmax(p2_logits), int(acc.sum()))
    assert ok, info
    assert (res["emit"][acc, 0] == x[acc]).all()
    # a rejected row's token follows the residual norm(max(p - q, 0))
    r = np.maximum(p - q, 0)
    r /= r.sum()
    ok, info = _band(np.bincount(res["emit"][~acc, 0], minlength=5), r, int((~acc).sum()))
    assert ok, info
    assert (res["pos_out"] == 100 + res["accept_len"] + 1).all()
    assert np.isfinite(res["gap"]).all() and (res["margin"] >= 0).all()


@pytest.mark.parametrize("seed", range(3))
def test_a_dense_q_with_few_nonzero_entries_is_the_sparse_case(seed):
    rng = np.random.default_rng(seed)
    B, kmax, V, NQ, T = 24, 5, 300, 4, 0.8
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    logits = rng.normal(0, 2.0, (R, V))
    q_tok = np.full((R, NQ), -1, np.int32)
    q_prob = np.zeros((R, NQ), np.float32)
    qd = np.zeros((R, V), np.float32)
    drafts = np.zeros((B, kmax), np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    for s in range(B):
        for j in range(k[s]):
            r = off[s] + j
            # supports near the target's top entries, so that drafts are often kept
            top = np.argsort(-logits[r])[:2 * NQ]
            supp = rng.choice(top, NQ, replace=False)
            w = rng.dirichlet(np.ones(NQ)).astype(np.float32)
            q_tok[r], q_prob[r] = supp, w
            qd[r, supp] = w
            drafts[s, j] = rng.choice(supp, p=w / w.sum())
    row_ctr = np.stack([np.arange(R) + 7, np.full(R, seed)], 1).astype(np.int32)
    pos = rng.integers(0, 1000, B).astype(np.int32)
    rows = oracle.sample_rows(logits, T, q_tok, q_prob, row_ctr, seed=555)
    sparse = oracle.sample_accept(drafts, kmax, k, None, 0, V, B, R, q_tok, q_prob, rows, row_ctr, 555, pos)
    dense = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, logits, T, qd, row_ctr, 555, pos)
    for key in ("status", "accept_len", "n_emit", "emit", "next_tok", "pos_out"):
        assert np.array_equal(sparse[key], dense[key]), key
    assert (dense["status"] == 0).all() and 0 < dense["accept_len"].sum() < k.sum()


def test_dense_error_paths_and_d2t():
    V, B, kmax = 6, 5, 2
    k = np.array([2, 1, 2, 0, 1], np.int32)
    R = int((k + 1).sum())
    logits = np.tile(np.array([0.0, 1.0, 2.0, 0.5, -1.0, 0.2]), (R, 1))
    qd = np.full((R, V), 1.0 / V, np.float32)
    qd[0, 4] = 0.0
    drafts = np.array([[4, 1], [2, 0], [9, 0], [0, 0], [1, 0]], np.int32)
    pos = np.array([10, 20, 30, 40, -1], np.int32)
    ctr = np.stack([np.arange(R), np.zeros(R)], 1).astype(np.int32)
    res = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R, logits, 1.0, qd, ctr, 3, pos)
    assert res["status"][0] == oracle.BAD_TOKEN          # zero draft mass
    assert res["status"][1] == 0
    assert res["status"][2] == oracle.BAD_TOKEN          # id outside the vocabulary
    assert res["status"][3] == 0 and res["accept_len"][3] == 0 and res["n_emit"][3] == 1
    assert res["status"][4] == oracle.BAD_POS
    flagged = res["status"] != 0
    assert (res["emit"][flagged] == -1).all() and (res["pos_out"][flagged] == pos[flagged]).all()
    bad = oracle.sample_accept_dense(drafts, kmax, k, None, 0, V, B, R + 1,
                                     np.vstack([logits, logits[:1]]), 1.0, np.vstack([qd, qd[:1]]),
                                     np.vstack([ctr, ctr[:1]]), 3, pos)
    assert (bad["status"] & oracle.BAD_ROWS).all()
    # d2t: draft-vocabulary ids mapped to target ids before the lookup of q
    d2t = np.array([5, 1, 2, 3, 0, 4], np.int32)
    via = oracle.sample_accept_dense(np.array([[1, 3]], np.int32), 2, np.array([2], np.int32), d2t, 6, V, 1, 3,
                                     logits[:3], 1.0, np.full((3, V), 1.0 / V, np.float32), ctr[:3], 3,
                                     np.array([0], np.int32))
    direct = oracle.sample_accept_dense(np.array([[1, 3]], np.int32), 2, np.array([2], np.int32), None, 0, V, 1, 3,
                                        logits[:3], 1.0, np.full((3, V), 1.0 / V, np.float32), ctr[:3], 3,
                                        np.array([0], np.int32))
    for key in ("status", "accept_len", "emit", "next_tok"):
        assert np.array_equal(via[key], direct[key]), key
