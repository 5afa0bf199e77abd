"""Adaptive draft depth, each quantity computed from its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): nothing in the product path
imports this module.

The trade-off is the one on the span-02 page (spec.rs, KPolicy: a smoothed
per-position acceptance estimate, a verify cost that grows with the rows, k chosen
for the least time per emitted token); oxinfer's DraftCosts (qwen_mtp.rs) weighs
the same two costs. The quantities, for draft positions j = 0, 1, ...:

  acceptance estimate   p_j = (kept_j + prior_p * prior_n) / (tried_j + prior_n)
                        (prior_n pseudo-observations at rate prior_p; a position is
                        tried when every earlier draft of its round was kept)
  all-kept probability  S_i = p_0 * p_1 * ... * p_{i-1},  S_0 = 1
  expected tokens       E(k) = S_0 + S_1 + ... + S_k   (kept drafts plus the bonus)
  verify cost           verify(r) = the polyline through (0, 0) and the measured
                        (rows, us) points, its last piece continued past the last
                        point
  cost per token        C(k; B) = (verify(B (k + 1)) + k * draft_us) / E(k)
  choice                the smallest k of least C over kmin .. kmax, the top lowered
                        to row_cap // B - 1 (never below kmin) when row_cap > 0
  observation           a round of k drafts with a kept: positions j < min(k, a + 1)
                        were tried, positions j < min(k, a) were kept
"""
from __future__ import annotations

import bisect
import math


class KPolicy:
    def __init__(self, kmin=1, kmax=6, prior_p=0.7, prior_n=8.0, draft_us=0.0, table=((1.0, 1.0),)):
        self.kmin, self.kmax = kmin, kmax
        self.prior_p, self.prior_n = prior_p, prior_n
        self.draft_us = draft_us
        # the polyline's corners: the origin, then the measured points
        self.corners = [(0.0, 0.0)] + [(float(r), float(t)) for r, t in table]
        self.tried = [0.0] * 64
        self.kept = [0.0] * 64

    def p(self, j):
        return (self.kept[j] + self.prior_p * self.prior_n) / (self.tried[j] + self.prior_n)

    def all_kept(self, i):
        return math.prod(self.p(j) for j in range(i))

    def expected_tokens(self, k):
        return sum(self.all_kept(i) for i in range(k + 1))

    def verify_cost(self, rows):
        r = float(rows)
        xs = [x for x, _ in self.corners]
        # the piece that ends at the first corner at or beyond r; before the origin
        # the first piece and past the last corner the last piece
        piece = min(max(bisect.bisect_left(xs, r), 1), len(xs) - 1)
        (x0, y0), (x1, y1) = self.corners[piece - 1], self.corners[piece]
        return y0 + (y1 - y0) * (r - x0) / (x1 - x0)

    def cost(self, k, B):
        return (self.verify_cost(B * (k + 1)) + k * self.draft_us) / self.expected_tokens(k)

    def choose(self, B, row_cap=0):
        top = self.kmax
        if row_cap > 0:
            top = min(top, max(row_cap // max(B, 1) - 1, self.kmin))
        return min(range(self.kmin, top + 1), key=lambda k: (self.cost(k, B), k))

    def update(self, k, accepted):
        for j in range(min(k, accepted + 1)):
            self.tried[j] += 1.0
        for j in range(min(k, accepted)):
            self.kept[j] += 1.0
