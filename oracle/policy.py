"""The adaptive draft-depth policy, written plainly (span-02 spec.rs KPolicy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

State: per draft position j, attempts att[j] and successes succ[j] (a position is
attempted when every earlier draft was kept, and succeeds when it is kept too).
    p_j        = (succ[j] + prior_p * prior_n) / (att[j] + prior_n)
    E(k)       = 1 + sum_{i=1..k} prod_{j<i} p_j          (tokens per sequence per cycle)
    verify(r)  = the piecewise-linear cost table at r rows (through the origin below the
                 first point, the last segment extended past the last point; a one-point
                 table is the line through the origin)
    cost(k; B) = (verify(B (k + 1)) + k * draft) / E(k)
    choose(B)  = the k in kmin .. min(kmax, row_cap / B - 1) with the least cost (the
                 smaller k on ties); without a row cap, kmin .. kmax
    update(k, a): for j < k: att[j] += 1 if j <= a; succ[j] += 1 if j < a
"""
from __future__ import annotations


class KPolicy:
    def __init__(self, kmin=1, kmax=6, prior_p=0.7, prior_n=8.0, draft_us=0.0, table=((1.0, 1.0),)):
        self.kmin, self.kmax = kmin, kmax
        self.prior_p, self.prior_n = prior_p, prior_n
        self.draft_us = draft_us
        self.table = [(float(r), float(t)) for r, t in table]
        self.att = [0.0] * 64
        self.succ = [0.0] * 64

    def p(self, j):
        return (self.succ[j] + self.prior_p * self.prior_n) / (self.att[j] + self.prior_n)

    def verify_cost(self, rows):
        t = self.table
        r = float(rows)
        if r <= t[0][0]:
            return t[0][1] * r / t[0][0]
        for (r0, c0), (r1, c1) in zip(t, t[1:]):
            if r <= r1:
                return c0 + (c1 - c0) * (r - r0) / (r1 - r0)
        if len(t) == 1:          # one point: the line through the origin continues
            return t[0][1] * r / t[0][0]
        (r0, c0), (r1, c1) = t[-2], t[-1]
        return c1 + (c1 - c0) * (r - r1) / (r1 - r0)

    def expected_tokens(self, k):
        e, prod = 1.0, 1.0
        for j in range(k):
            prod *= self.p(j)
            e += prod
        return e

    def cost(self, k, B):
        return (self.verify_cost(B * (k + 1)) + (k * self.draft_us if k > 0 else 0.0)) / self.expected_tokens(k)

    def choose(self, B, row_cap=0):
        hi = self.kmax
        if row_cap > 0:
            hi = min(hi, max(row_cap // max(B, 1) - 1, self.kmin))
        best, best_cost = self.kmin, float("inf")
        for k in range(self.kmin, hi + 1):
            c = self.cost(k, B)
            if c < best_cost:
                best, best_cost = k, c
        return best

    def update(self, k, accepted):
        for j in range(k):
            if j <= accepted:
                self.att[j] += 1.0
            if j < accepted:
                self.succ[j] += 1.0
