"""Pins of the oracle's greedy acceptance with stop tokens and a generation limit
(oxinfer step: an accepted stop token ends the round, the committed tokens end at
the first stop token, the session advances by the number committed; DSSD _commit:
truncation at a stop token or at max_new; DSSD generate_ar: one-row decoding stops
after the same token), CPU only."""
import numpy as np
import pytest

import oracle
from oracle.toy_lm import ToyLM


def _round_like_oxinfer(g, drafts, stops, remaining):
    """One round written the way oxinfer's step reads: accept while the draft equals the
    row's greedy token, break after an accepted stop token, else take the row's token and
    break; the bonus only if every draft was kept and the last kept one is no stop token;
    then truncate after the first stop token and at the limit."""
    out = []
    for j, d in enumerate(drafts):
        if d == g[j]:
            out.append(d)
            if d in stops:
                break
        else:
            out.append(g[j])
            break
    else:
        if not (out and out[-1] in stops):
            out.append(g[len(drafts)])
    for i, t in enumerate(out):
        if t in stops:
            out = out[:i + 1]
            break
    if remaining is not None:
        out = out[:remaining]
    return out


@pytest.mark.parametrize("seed", range(4))
def test_stop_rule_matches_the_round_written_out(seed):
    rng = np.random.default_rng(seed)
    B, kmax, V = 300, 6, 8
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)])
    drafts = np.full((B, kmax), -1, np.int32)
    for s in range(B):
        for j in range(k[s]):
            drafts[s, j] = g[off[s] + j] if rng.uniform() < 0.75 else rng.integers(0, V)
    stops = [2, 5]
    remaining = rng.integers(1, 8, B).astype(np.int32) if seed % 2 else None
    pos = rng.integers(0, 50, B).astype(np.int32)
    r = oracle.greedy_accept_stop(g, drafts, kmax, k, None, 0, V, B, R, stops, remaining, pos)
    assert (r["status"] == 0).all()
    for s in range(B):
        want = _round_like_oxinfer(list(g[off[s]:off[s + 1]]), list(drafts[s, :k[s]]), stops,
                                   None if remaining is None else int(remaining[s]))
        c = len(want)
        assert list(r["emit"][s, :c]) == want and (r["emit"][s, c:] == -1).all()
        assert r["n_emit"][s] == c and r["pos_out"][s] == pos[s] + c and r["next_tok"][s] == want[-1]
        kept = 0
        while kept < min(k[s], c) and drafts[s, kept] == g[off[s] + kept]:
            kept += 1
        assert r["accept_len"][s] == kept
        lim = remaining is not None and c == remaining[s]
        assert r["done"][s] == int(want[-1] in stops or lim)


def test_stop_hand_cases():
    # drafts [3, 2, 4] against g [3, 2, 4, 7]; stop token 2 accepted at draft 1
    g = np.array([3, 2, 4, 7], np.int32)
    d = np.array([[3, 2, 4]], np.int32)
    one = lambda stops, rem=None: oracle.greedy_accept_stop(g, d, 3, np.array([3], np.int32), None, 0, 10, 1, 4,
                                                             stops, rem, np.array([100], np.int32))
    r = one([2])
    assert list(r["emit"][0]) == [3, 2, -1, -1] and r["n_emit"][0] == 2 and r["accept_len"][0] == 2
    assert r["pos_out"][0] == 102 and r["next_tok"][0] == 2 and r["done"][0] == 1
    r = one([7])                                        # the bonus is the stop token
    assert list(r["emit"][0]) == [3, 2, 4, 7] and r["done"][0] == 1 and r["pos_out"][0] == 104
    r = one([9])                                        # no stop: the plain greedy round
    assert r["n_emit"][0] == 4 and r["done"][0] == 0
    r = one([9], np.array([2], np.int32))               # the limit cuts after two tokens
    assert list(r["emit"][0]) == [3, 2, -1, -1] and r["done"][0] == 1 and r["accept_len"][0] == 2
    r = one([9], np.array([0], np.int32))
    assert r["status"][0] == oracle.BAD_LIMIT and r["n_emit"][0] == 0 and r["pos_out"][0] == 100
    # a rejected draft that is a stop token stops nothing: the row's own token is emitted
    r = oracle.greedy_accept_stop(g, np.array([[3, 5, 4]], np.int32), 3, np.array([3], np.int32), None, 0, 10, 1,
                                  4, [5], None, np.array([0], np.int32))
    assert list(r["emit"][0]) == [3, 2, -1, -1] and r["done"][0] == 0


def test_toy_spec_with_stop_ends_where_one_row_decoding_ends():
    """DSSD generate_ar and generate_spec share the stop rule, so both streams end at the
    same token; with the limit alone both give exactly max_new tokens."""
    m = ToyLM(seed=0)
    prompt = list(np.random.default_rng(1).integers(0, m.V, 20))
    free = m.generate_ar(prompt, 60)
    stop = free[23]                                    # a token the stream emits
    ref = m.generate_ar(prompt, 60, stop_ids=(stop,))
    assert ref[-1] == stop and len(ref) <= 24
    rng = np.random.default_rng(7)

    def drafter(out, kk):
        true = free[len(out):len(out) + kk]
        true = true + [0] * (kk - len(true))
        return [t if rng.uniform() >= 0.2 else int((t + 1) % m.V) for t in true]

    out, _ = m.generate_spec(prompt, 60, drafter, 4, stop_ids=(stop,))
    assert out == ref
    out, _ = m.generate_spec(prompt, 37, drafter, 4, stop_ids=())
    assert out == free[:37]


def test_truncation_of_a_tree_walk_keeps_only_committed_path_nodes():
    """Walk: root -> node 2 (token 7) -> node 3 (token 5), bonus 9; stop token 7 ends the
    round after node 2, so the path keeps node 2 only and pos advances by one."""
    g = np.array([7, 1, 5, 9], np.int32)                 # greedy tokens of nodes 0..3
    drafts = np.array([[4, 7, 5]], np.int32)             # nodes 1..3
    parent = np.array([[-1, 0, 0, 2]], np.int32)
    res = oracle.tree_accept(g, drafts, 3, np.array([3], np.int32), parent, None, 0, 10, 1, 4,
                             np.array([50], np.int32))
    assert list(res["path"][0]) == [2, 3, -1] and list(res["emit"][0]) == [7, 5, 9, -1]
    t = oracle.truncate_stop(res, 3, [7], None, np.array([50], np.int32), path=res["path"])
    assert list(t["path"][0]) == [2, -1, -1] and list(t["emit"][0]) == [7, -1, -1, -1]
    assert t["accept_len"][0] == 1 and t["n_emit"][0] == 1 and t["pos_out"][0] == 51 and t["done"][0] == 1
    assert t["next_tok"][0] == 7
    t = oracle.truncate_stop(res, 3, [], np.array([2], np.int32), np.array([50], np.int32), path=res["path"])
    assert list(t["path"][0]) == [2, 3, -1] and t["n_emit"][0] == 2 and t["accept_len"][0] == 2
    assert t["done"][0] == 1 and t["next_tok"][0] == 5


def test_toy_tree_with_stop_ends_where_one_row_decoding_ends():
    m = ToyLM(seed=0)
    prompt = list(np.random.default_rng(1).integers(0, m.V, 20))
    free = m.generate_ar(prompt, 60)
    stop = free[29]
    ref = m.generate_ar(prompt, 60, stop_ids=(stop,))
    assert ref[-1] == stop
    rng = np.random.default_rng(4)

    def drafter(out):
        true = free[len(out):len(out) + 6] + [0] * 6
        par, toks, spine = [], [], [0]
        for d in range(4):
            par.append(spine[-1])
            toks.append(true[d] if rng.uniform() < 0.8 else int((true[d] + 1) % m.V))
            spine.append(len(toks))
            par.append(spine[-2])                        # a sibling holding the other choice
            toks.append(true[d] if toks[-1] != true[d] else int((true[d] + 2) % m.V))
        return par, toks

    out, _ = m.generate_tree(prompt, 60, drafter, stop_ids=(stop,))
    assert out == ref
    out, _ = m.generate_tree(prompt, 41, drafter, stop_ids=())
    assert out == free[:41]


@pytest.mark.parametrize("seed", range(4))
def test_truncation_is_idempotent_and_matches_the_combined_greedy_call(seed):
    """Truncating a greedy round equals the fused stop call, and truncating the result
    again changes nothing (its last token is already the first stop, and its length is
    already within the limit)."""
    rng = np.random.default_rng(seed)
    B, kmax, V = 12, 6, 40
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    g = rng.integers(0, V, R).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(k + 1)[:-1]])
    drafts = np.zeros((B, kmax), np.int32)
    for s in range(B):
        a = rng.integers(0, k[s] + 1)
        drafts[s, :k[s]] = rng.integers(0, V, k[s])
        drafts[s, :a] = g[off[s]:off[s] + a]
    pos = rng.integers(0, 100, B).astype(np.int32)
    stops = list(rng.choice(g, 3, replace=False))
    rem = rng.integers(1, kmax + 3, B).astype(np.int32)
    base = oracle.greedy_accept(g, drafts, kmax, k, None, 0, V, B, R, pos)
    t1 = oracle.truncate_stop(base, kmax, stops, rem, pos)
    fused = oracle.greedy_accept_stop(g, drafts, kmax, k, None, 0, V, B, R, stops, rem, pos)
    for key in ("emit", "n_emit", "accept_len", "next_tok", "pos_out", "done", "status"):
        assert np.array_equal(t1[key], fused[key]), key
    t2 = oracle.truncate_stop(t1, kmax, stops, rem, pos)
    for key in ("emit", "n_emit", "accept_len", "next_tok", "pos_out", "done", "status"):
        assert np.array_equal(t1[key], t2[key]), key


def test_truncation_flags_outputs_that_are_no_round():
    """n_emit outside 1..kmax+1 or accept_len outside 0..n_emit: BAD_ROWS, flagged
    outputs; a sequence flagged on entry is left untouched with done 0."""
    kmax = 3
    res = {
        "emit": np.array([[5, -1, -1, -1], [5, 6, -1, -1], [5, 6, 7, 8], [-1, -1, -1, -1]], np.int32),
        "n_emit": np.array([0, 2, 4, 0], np.int32),
        "accept_len": np.array([0, 3, 3, -1], np.int32),
        "next_tok": np.array([5, 6, 8, -1], np.int32),
        "pos_out": np.array([10, 12, 14, 10], np.int32),
        "status": np.array([0, 0, 0, oracle.BAD_TOKEN], np.int32),
    }
    pos = np.array([10, 10, 10, 10], np.int32)
    t = oracle.truncate_stop(res, kmax, [99], None, pos)
    assert list(t["status"]) == [oracle.BAD_ROWS, oracle.BAD_ROWS, 0, oracle.BAD_TOKEN]
    assert list(t["n_emit"]) == [0, 0, 4, 0] and list(t["pos_out"]) == [10, 10, 14, 10]
    assert list(t["done"]) == [0, 0, 0, 0]
    assert (t["emit"][:2] == -1).all() and list(t["accept_len"][:2]) == [-1, -1]
