"""The lossless invariant, checked on the oracle with a toy one-layer model.

The span-02 spec.rs module doc, the DSSD fast.py generate_ar baseline and the
oxinfer / flashrt exactness notes all state it: greedy speculative decoding emits
exactly the one-row greedy stream, whatever the drafts. A wrong acceptance rule,
a wrong bonus token, a wrong position advance or attention that sees a key past
its row's position all break it.
"""
import numpy as np
import pytest

from oracle.toy_lm import ToyLM

N_NEW = 96


@pytest.fixture(scope="module")
def toy():
    m = ToyLM(seed=0)
    prompt = list(np.random.default_rng(1).integers(0, m.V, 20))
    ref = m.generate_ar(prompt, N_NEW + 8)
    return m, prompt, ref


@pytest.mark.parametrize("kind,k", [("perfect", 3), ("corrupt", 3), ("random", 3), ("corrupt", 6),
                                    ("perfect", 1)])
def test_spec_stream_equals_one_row_greedy(toy, kind, k):
    m, prompt, ref = toy
    rng = np.random.default_rng(7)

    def drafter(out, kk):
        n = len(out)
        true = ref[n:n + kk]
        true = true + [0] * (kk - len(true))
        if kind == "perfect":
            return true
        if kind == "random":
            return list(rng.integers(0, m.V, kk))
        return [t if rng.uniform() >= 0.3 else int((t + 1 + rng.integers(0, m.V - 1)) % m.V) for t in true]

    out, hist = m.generate_spec(prompt, N_NEW, drafter, k)
    assert out == ref[:N_NEW]
    if kind == "perfect":
        assert min(hist[:-1]) == k          # every draft accepted (the tail may run past ref)
    if kind == "random":
        assert np.mean(hist) < 0.2


def test_invariant_detects_a_wrong_bonus(toy):
    """Sanity of the test itself: emitting the draft instead of the target token at the
    first mismatch breaks the stream."""
    m, prompt, ref = toy
    rng = np.random.default_rng(3)
    bad = ref[1:4]
    bad = [bad[0], (bad[1] + 5) % m.V, bad[2]]
    import oracle
    g = m.generate_ar(prompt, 4)
    assert g == ref[:4]
    res = oracle.greedy_accept(np.array(ref[:4], np.int32), np.array([bad], np.int32), 3,
                               np.array([3], np.int32), None, 0, m.V, 1, 4, np.array([0], np.int32))
    assert list(res["emit"][0, :res["n_emit"][0]]) != ref[:1] + bad
