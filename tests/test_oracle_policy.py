"""Pins of the draft-depth policy oracle (span-02 spec.rs KPolicy), CPU only:
closed forms of its pieces and the behaviour its definition implies."""
import math

import numpy as np
import pytest

from oracle.policy import KPolicy


def test_expected_tokens_geometric_closed_form():
    """With no observations every p_j is prior_p, so E(k) = (1 - p^(k+1)) / (1 - p)."""
    for p in (0.3, 0.7, 0.95):
        pol = KPolicy(prior_p=p, prior_n=8.0)
        for k in range(8):
            assert math.isclose(pol.expected_tokens(k), (1 - p ** (k + 1)) / (1 - p), rel_tol=1e-12)


def test_acceptance_estimate_is_the_smoothed_rate():
    pol = KPolicy(prior_p=0.5, prior_n=4.0)
    for a in (0, 1, 3, 3, 3, 4):       # rounds of k = 4 drafts with a kept
        pol.update(4, a)
    # position j is attempted when a >= j and kept when a > j
    assert pol.tried[:4] == [6, 5, 4, 4] and pol.kept[:4] == [5, 4, 4, 1]
    assert math.isclose(pol.p(0), (5 + 2) / (6 + 4)) and math.isclose(pol.p(3), (1 + 2) / (4 + 4))
    assert pol.tried[4] == 0


def test_verify_cost_interpolates_the_table():
    pol = KPolicy(table=[(16, 200.0), (32, 210.0), (64, 250.0)])
    assert pol.verify_cost(16) == 200.0 and pol.verify_cost(64) == 250.0
    assert math.isclose(pol.verify_cost(8), 100.0)             # through the origin below the first point
    assert math.isclose(pol.verify_cost(48), 230.0)
    assert math.isclose(pol.verify_cost(96), 290.0)            # the last segment extended


def test_choose_extremes():
    table = [(16, 200.0), (128, 260.0)]
    # free drafts and sure acceptance: the deepest allowed k
    pol = KPolicy(kmin=1, kmax=7, prior_p=0.99, prior_n=1e9, draft_us=0.0, table=table)
    assert pol.choose(16) == 7
    assert pol.choose(16, row_cap=64) == 3                     # 16 (k + 1) <= 64
    # drafts that always fail and cost something: the shallowest k
    pol = KPolicy(kmin=1, kmax=7, prior_p=0.01, prior_n=1e9, draft_us=30.0, table=table)
    assert pol.choose(16) == 1


def test_choose_is_the_brute_force_minimum():
    rng = np.random.default_rng(3)
    for _ in range(200):
        pts = np.sort(rng.uniform(1, 200, 4))
        cost = np.cumsum(rng.uniform(1, 50, 4))
        pol = KPolicy(kmin=int(rng.integers(0, 2)), kmax=int(rng.integers(2, 9)), prior_p=rng.uniform(0.1, 0.95),
                      prior_n=rng.uniform(1, 10), draft_us=rng.uniform(0, 20), table=list(zip(pts, cost)))
        for _ in range(int(rng.integers(0, 30))):
            k = int(rng.integers(1, 9))
            pol.update(k, int(rng.integers(0, k + 1)))
        B = int(rng.integers(1, 33))
        costs = {k: pol.cost(k, B) for k in range(pol.kmin, pol.kmax + 1)}
        want = min(costs, key=lambda k: (costs[k], k))
        assert pol.choose(B) == want
