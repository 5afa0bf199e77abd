"""Pins of the oracle's speculative-sampling verify, CPU only.

DSSD fast.py _sample_verify and oxinfer speculative_accept:
  * draft x is accepted with probability min(1, p(x)/q(x));
  * at the first rejection the token is drawn from norm(max(p - q, 0));
  * if every draft is accepted, the bonus is drawn from p.
memra's sampled-spec note asks for counter-based Philox randomness.

The pins:
  * the generator against the Philox4x32-10 known-answer vectors published with
    the Random123 library (kat_vectors, philox4x32_10 lines);
  * Gumbel-max draws against the softmax and residual probabilities
    (binomial 5-sigma bands);
  * the theorem the method rests on: the emitted token is distributed as the
    target p, whatever q;
  * the zero-temperature limit, which must reduce to greedy acceptance.
"""
import numpy as np
import pytest

import oracle

# Random123 kat_vectors: philox4x32 10 rounds, counter, key -> output
PHILOX_KAT = [
    ([0x00000000, 0x00000000, 0x00000000, 0x00000000], [0x00000000, 0x00000000],
     [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
    ([0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff], [0xffffffff, 0xffffffff],
     [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
    ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
     [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert list(oracle.philox4x32_10(ctr, key)) == want


def _softmax(z):
    e = np.exp(z - z.max())
    return e / e.sum()


def _band(counts, probs, n, sigmas=5.0):
    """Every category's count within `sigmas` binomial standard deviations."""
    exp = probs * n
    sd = np.sqrt(n * probs * (1 - probs)) + 1e-9
    return np.all(np.abs(counts - exp) <= sigmas * sd + 1), (counts, exp)


def test_gumbel_max_draws_follow_softmax_and_residual():
    V, N, T = 7, 60000, 0.7
    logits = np.array([1.0, 0.2, -0.5, 2.0, 0.0, 1.5, -2.0])
    q_tok = np.array([[3, 5, 0, -1]], np.int32)
    q_prob = np.array([[0.5, 0.3, 0.2, 0.0]], np.float32)
    L = np.tile(logits, (N, 1))
    ctr = np.stack([np.arange(N), np.full(N, 11)], 1).astype(np.int32)
    out = oracle.sample_rows(L, T, np.tile(q_tok, (N, 1)), np.tile(q_prob, (N, 1)), ctr, seed=0x1234_5678_9abc)
    p = _softmax(logits / T)
    ok, info = _band(np.bincount(out["sample_p"], minlength=V), p, N)
    assert ok, info
    q = np.zeros(V)
    q[[3, 5, 0]] = [0.5, 0.3, 0.2]
    r = np.maximum(p - q, 0)
    r /= r.sum()
    ok, info = _band(np.bincount(out["sample_res"], minlength=V), r, N)
    assert ok, info
    assert (out["sample_res"] != 3).all() == (r[3] == 0)
    np.testing.assert_allclose(out["lse"], np.log(np.exp(logits / T).sum()), rtol=1e-12)
    np.testing.assert_allclose(out["z_supp"][0, :3], logits[[3, 5, 0]] / T, rtol=1e-15)
    assert np.isnan(out["z_supp"][0, 3])


def _one_draft_batch(B, p_logits, p2_logits, q, rng, T=1.0, support=None):
    """B sequences, one draft each, drawn from q; returns the emitted tokens. The
    support list is q's nonzero entries, or support = (tokens, masses), whose masses
    summed per token must give q (a token may appear in several entries)."""
    V = len(p_logits)
    x = rng.choice(V, size=B, p=q)
    if support is None:
        supp = np.nonzero(q)[0]
        masses = q[supp]
    else:
        supp, masses = (np.asarray(a) for a in support)
        summed = np.zeros(V)
        np.add.at(summed, supp, masses)
        np.testing.assert_allclose(summed, q)
    NQ = len(supp)
    R = 2 * B
    logits = np.empty((R, V))
    logits[0::2] = p_logits
    logits[1::2] = p2_logits
    q_tok = np.full((R, NQ), -1, np.int32)
    q_prob = np.zeros((R, NQ), np.float32)
    q_tok[0::2] = supp
    q_prob[0::2] = masses
    row_ctr = np.stack([np.repeat(np.arange(B), 2) * 0 + np.tile([100, 101], B), np.repeat(np.arange(B), 2)],
                       1).astype(np.int32)
    rows = oracle.sample_rows(logits, T, q_tok, q_prob, row_ctr, seed=99)
    res = oracle.sample_accept(x[:, None], 1, np.ones(B, np.int32), None, 0, V, B, R, q_tok, q_prob, rows,
                               row_ctr, 99, np.full(B, 100, np.int32))
    assert (res["status"] == 0).all()
    return x, res


@pytest.mark.parametrize("q", [np.array([0.5, 0.0, 0.3, 0.2, 0.0]),      # overlaps p loosely
                               np.array([0.0, 1.0, 0.0, 0.0, 0.0]),      # a point mass
                               np.array([0.2, 0.2, 0.2, 0.2, 0.2])])     # uniform
def test_speculative_sampling_emits_the_target_distribution(q):
    """The theorem behind the method: the first emitted token ~ p(row 0), whatever q
    is; after an accepted draft the next one ~ p(row 1)."""
    rng = np.random.default_rng(5)
    B = 60000
    p_logits = np.array([0.3, 1.2, -0.4, 0.8, 0.0])
    p2_logits = np.array([-1.0, 0.0, 2.0, 0.5, 0.1])
    x, res = _one_draft_batch(B, p_logits, p2_logits, q, rng)
    first = res["emit"][:, 0]
    ok, info = _band(np.bincount(first, minlength=5), _softmax(p_logits), B)
    assert ok, info
    acc = res["accept_len"] == 1
    assert (res["n_emit"] == res["accept_len"] + 1).all()
    ok, info = _band(np.bincount(res["emit"][acc, 1], minlength=5), _softmax(p2_logits), int(acc.sum()))
    assert ok, info
    # acceptance rate = sum_x min(p(x), q(x))
    p = _softmax(p_logits)
    rate = np.minimum(p, q).sum()
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / B)
    assert (res["emit"][acc, 0] == x[acc]).all()
    assert (res["pos_out"] == 100 + res["accept_len"] + 1).all()


def test_duplicated_support_entries_still_emit_the_target_distribution():
    """A token listed in several support entries has q = the entries' summed mass,
    in the keep test as in the residual; keeping it with probability p / (one
    entry's mass) instead would raise its acceptance rate and bias the emitted
    tokens away from p."""
    rng = np.random.default_rng(6)
    B = 60000
    p_logits = np.array([0.3, 1.2, -0.4, 0.8, 0.0])
    p2_logits = np.array([-1.0, 0.0, 2.0, 0.5, 0.1])
    q = np.array([0.5, 0.0, 0.3, 0.2, 0.0])
    support = ([0, 2, 0, 3], [0.25, 0.3, 0.25, 0.2])
    x, res = _one_draft_batch(B, p_logits, p2_logits, q, rng, support=support)
    ok, info = _band(np.bincount(res["emit"][:, 0], minlength=5), _softmax(p_logits), B)
    assert ok, info
    acc = res["accept_len"] == 1
    p = _softmax(p_logits)
    kept0 = acc[x == 0].mean()
    want0 = min(1.0, p[0] / q[0])
    assert abs(kept0 - want0) < 5 * np.sqrt(want0 * (1 - want0) / (x == 0).sum())
    rate = np.minimum(p, q).sum()
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / B)
    ok, info = _band(np.bincount(res["emit"][acc, 1], minlength=5), _softmax(p2_logits), int(acc.sum()))
    assert ok, info


def test_zero_temperature_reduces_to_greedy_acceptance():
    """T -> 0 with point-mass drafts: p is one-hot at the argmax, so a draft is kept iff
    it is the argmax and the emitted token is the argmax (oxinfer speculative_accept's
    doc) -- the chain walk must then equal the greedy oracle's, sequence for sequence."""
    rng = np.random.default_rng(9)
    B, kmax, V = 200, 5, 50
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    logits = rng.standard_normal((R, V)) * 3
    g = logits.argmax(1).astype(np.int32)
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
    pos = rng.integers(0, 1000, B).astype(np.int32)
    rows = oracle.sample_rows(logits, 1e-4, q_tok, q_prob, row_ctr, seed=3)
    assert (rows["sample_p"] == g).all()
    a = oracle.sample_accept(drafts, kmax, k, None, 0, V, B, R, q_tok, q_prob, rows, row_ctr, 3, pos)
    b = oracle.greedy_accept(g, drafts, kmax, k, None, 0, V, B, R, pos)
    for key in ("pos_out", "accept_len", "n_emit", "emit", "next_tok", "status"):
        np.testing.assert_array_equal(a[key], b[key])
    assert 0 < a["accept_len"].mean() < kmax


def test_accept_probability_of_a_point_mass_is_p():
    """q = point mass at x: the draft is kept with probability p(x)."""
    B, V = 40000, 6
    logits = np.array([0.0, 1.0, 0.5, -0.5, 0.2, 0.9])
    p = _softmax(logits)
    x, res = _one_draft_batch(B, logits, logits, np.eye(V)[1], np.random.default_rng(2))
    rate = (res["accept_len"] == 1).mean()
    assert abs(rate - p[1]) < 5 * np.sqrt(p[1] * (1 - p[1]) / B)
    rej = res["accept_len"] == 0
    assert (res["emit"][rej, 0] != 1).all()      # the residual excludes the rejected point mass


def test_sample_accept_error_paths():
    V, B = 10, 3
    k = np.array([2, 1, 1], np.int32)
    R = 7
    logits = np.zeros((R, V))
    drafts = np.array([[1, 2], [3, -1], [4, -1]], np.int32)
    q_tok = np.array([[1], [2], [-1], [5], [-1], [4], [-1]], np.int32)   # sequence 1's draft 3 is not in its support
    q_prob = np.array([[1], [1], [0], [1], [0], [1], [0]], np.float32)
    row_ctr = np.zeros((R, 2), np.int32)
    rows = oracle.sample_rows(logits, 1.0, q_tok, q_prob, row_ctr, 0)
    pos = np.array([5, 5, -1], np.int32)
    r = oracle.sample_accept(drafts, 2, k, None, 0, V, B, R, q_tok, q_prob, rows, row_ctr, 0, pos)
    assert list(r["status"]) == [0, oracle.BAD_TOKEN, oracle.BAD_POS]
    assert list(r["accept_len"][1:]) == [-1, -1] and list(r["pos_out"]) == [5 + r["accept_len"][0] + 1, 5, -1]
    r = oracle.sample_accept(drafts, 2, k, None, 0, V, B, R + 1, q_tok, q_prob, rows, row_ctr, 0, pos)
    assert (r["status"] & oracle.BAD_ROWS).all()
