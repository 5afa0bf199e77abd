"""The library's draft-depth policy (host C, spec_kpolicy_*) against the oracle's
(span-02 spec.rs KPolicy), CPU only: the same k on random tables and histories,
the same estimates to 1e-12, and the argument checks."""
import numpy as np
import pytest

import greedy_draft_verify_amd as gdv
from oracle.policy import KPolicy as OraclePolicy


def _pair(rng):
    n = int(rng.integers(1, 8))
    rows = np.sort(rng.choice(np.arange(1, 400), n, replace=False)).astype(float)
    us = np.sort(rng.uniform(50, 600, n))
    kw = dict(kmin=int(rng.integers(0, 3)), kmax=int(rng.integers(3, 12)), prior_p=float(rng.uniform(0.05, 1.0)),
              prior_n=float(rng.uniform(0.5, 20)), draft_us=float(rng.uniform(0, 40)), table=list(zip(rows, us)))
    return gdv.KPolicy(**kw), OraclePolicy(**kw)


@pytest.mark.parametrize("seed", range(5))
def test_policy_matches_the_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        lib, ref = _pair(rng)
        for _ in range(int(rng.integers(0, 40))):
            k = int(rng.integers(0, 12))
            a = int(rng.integers(0, k + 1))
            lib.update(k, a)
            ref.update(k, a)
        for j in range(12):
            assert abs(lib.p(j) - ref.p(j)) <= 1e-12
        for r in (0.5, 1, 7, 16, 80, 250, 399, 800):
            assert abs(lib.verify_cost(r) - ref.verify_cost(r)) <= 1e-9 * max(1.0, abs(ref.verify_cost(r)))
        for k in range(12):
            assert abs(lib.expected_tokens(k) - ref.expected_tokens(k)) <= 1e-12 * ref.expected_tokens(k)
        for B in (1, 4, 16, 64):
            for cap in (0, 16, 128):
                assert lib.choose(B, cap) == ref.choose(B, cap)


def test_batch_update_skips_flagged_sequences():
    rng = np.random.default_rng(9)
    lib, ref = _pair(rng)
    k = np.array([4, 4, 2, 6], np.int32)
    a = np.array([2, -1, 2, 0], np.int32)
    lib.update_batch(k, a)
    for kk, aa in zip(k, a):
        if aa >= 0:
            ref.update(int(kk), int(aa))
    assert list(lib.st.tried[:8]) == ref.tried[:8] and list(lib.st.kept[:8]) == ref.kept[:8]


def test_policy_argument_checks():
    with pytest.raises(gdv.SpecError):
        gdv.KPolicy(kmin=3, kmax=2)
    with pytest.raises(gdv.SpecError):
        gdv.KPolicy(kmax=64)
    with pytest.raises(gdv.SpecError):
        gdv.KPolicy(prior_p=0.0)
    with pytest.raises(gdv.SpecError):
        gdv.KPolicy(table=[(16, 100.0), (16, 120.0)])
    with pytest.raises(gdv.SpecError):
        gdv.KPolicy(table=[(16, -1.0)])
    assert gdv.lib().spec_kpolicy_choose(None, 4, 0) == -1
