"""A toy one-layer language model driven through the oracle, for the lossless invariant.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The span-02 spec.rs module doc states the invariant the whole verify step exists
for: a token is emitted only if it equals the target's greedy token at the verify
row before it, and rows are computed exactly as one-row decoding computes them, so
the emitted stream equals one-row greedy decoding. The DSSD fast.py page measures
against its one-row ``generate_ar`` stream the same way.

The toy model (sizes of the tiny workload): token x at position p
    e = E[x]                                      bf16 embedding, H = 256
    q = bf16(Wq e), k = bf16(Wk e), v = bf16(Wv e) 4 query heads / 1 kv head, D = 64
    k, v appended into the paged pool at p; attention over positions 0..p
    h = bf16(e + Wo bf16(attn))
    greedy token = argmax(Wlm h)                  vocabulary 1024
Projections are fp64 matrix-vector products of bf16 values, one row at a time, so a
row's arithmetic never depends on how many rows share a call.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

PAGE = 16


class ToyLM:
    def __init__(self, seed=0, V=1024, H=256, Hq=4, Hkv=1, D=64, max_len=1024):
        rng = np.random.default_rng(seed)
        bfr = lambda shape, std: oracle.f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
        self.V, self.H, self.Hq, self.Hkv, self.D = V, H, Hq, Hkv, D
        self.E = bfr((V, H), 1.0)
        self.Wq = bfr((Hq * D, H), 1 / math.sqrt(H))
        self.Wk = bfr((Hkv * D, H), 1 / math.sqrt(H))
        self.Wv = bfr((Hkv * D, H), 1 / math.sqrt(H))
        self.Wo = bfr((H, Hq * D), 1 / math.sqrt(Hq * D))
        self.Wlm = bfr((V, H), 1 / math.sqrt(H))
        self.f = {n: oracle.bf16_bits_to_f64(getattr(self, n)) for n in ("E", "Wq", "Wk", "Wv", "Wo")}
        self.max_pages = max_len // PAGE
        # pages of the single sequence, scattered over a larger pool
        self.n_pages = self.max_pages * 2
        self.page_table = rng.permutation(self.n_pages)[: self.max_pages].astype(np.int32)[None, :]
        self.reset()

    def reset(self):
        self.k_pool = np.zeros((self.n_pages, self.Hkv, PAGE * self.D), np.uint16)
        self.v_pool = np.zeros((self.n_pages, self.Hkv, PAGE * self.D), np.uint16)

    def _proj(self, W, x):
        return oracle.f32_to_bf16_bits(np.array([W[i] @ x for i in range(W.shape[0])], np.float64).astype(np.float32))

    def forward_rows(self, tokens, pos, parent=None):
        """Rows tokens[j] at positions pos + j (one sequence), or, with ``parent``, the
        nodes of a draft tree in creation order (row j writes slot pos + j and attends
        to slots 0..pos plus its own path). Returns greedy tokens [T]."""
        T = len(tokens)
        q = np.empty((T, self.Hq, self.D), np.uint16)
        kn = np.empty((T, self.Hkv, self.D), np.uint16)
        vn = np.empty((T, self.Hkv, self.D), np.uint16)
        for j, x in enumerate(tokens):
            e = self.f["E"][x]
            q[j] = self._proj(self.f["Wq"], e).reshape(self.Hq, self.D)
            kn[j] = self._proj(self.f["Wk"], e).reshape(self.Hkv, self.D)
            vn[j] = self._proj(self.f["Wv"], e).reshape(self.Hkv, self.D)
        posa = np.array([pos], np.int32)
        ka = np.array([T - 1], np.int32)
        off, st = oracle.validate(self.page_table, self.max_pages, self.n_pages, posa, ka, 64, 1, T)
        assert st[0] == 0
        oracle.append_kv(kn, vn, self.k_pool, self.v_pool, self.page_table, self.max_pages, posa, ka, off,
                         st, 1, self.Hkv, self.D)
        if parent is None:
            att = oracle.verify_attn(q, self.k_pool, self.v_pool, self.page_table, self.max_pages, posa, ka,
                                     off, st, 1, T, self.Hq, self.Hkv, self.D, 1 / math.sqrt(self.D))
        else:
            att = oracle.verify_attn_tree(q, self.k_pool, self.v_pool, self.page_table, self.max_pages, posa,
                                          ka, np.asarray(parent, np.int32)[None, :], T - 1, off, st, 1, T,
                                          self.Hq, self.Hkv, self.D, 1 / math.sqrt(self.D))
        att_bf = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(att.astype(np.float32)))
        h = np.empty((T, self.H), np.uint16)
        for j, x in enumerate(tokens):
            hv = self.f["E"][x] + np.array([self.f["Wo"][i] @ att_bf[j].reshape(-1) for i in range(self.H)])
            h[j] = oracle.f32_to_bf16_bits(hv.astype(np.float32))
        g, _, _, _ = oracle.lm_head_argmax(h, self.Wlm, T, self.H, self.V)
        return g

    def generate_ar(self, prompt, n_new, stop_ids=()):
        """One-row greedy decoding (DSSD fast.py generate_ar): n_new tokens, or fewer
        when a stop token is emitted (it is kept, and nothing follows it)."""
        self.reset()
        out = []
        g = None
        for i, x in enumerate(prompt):
            g = int(self.forward_rows([x], i)[0])
        pos = len(prompt)
        while len(out) < n_new:
            out.append(g)
            if g in stop_ids:
                break
            g = int(self.forward_rows([g], pos)[0])
            pos += 1
        return out

    def generate_spec(self, prompt, n_new, drafter, k, stop_ids=None):
        """Draft -> one verify of k+1 rows -> greedy accept -> pos += a + 1. With
        stop_ids, the acceptance truncates at the first stop token and at the tokens
        still allowed (n_new minus those emitted), and generation ends when it says so."""
        self.reset()
        for i, x in enumerate(prompt[:-1]):
            self.forward_rows([x], i)
        x0, pos = prompt[-1], len(prompt) - 1
        out, accepted_hist = [], []
        while len(out) < n_new:
            drafts = [int(d) for d in drafter(out, k)]
            g = self.forward_rows([x0] + drafts, pos)
            args = (g, np.array([drafts], np.int32), k, np.array([k], np.int32), None, 0, self.V, 1, k + 1)
            if stop_ids is None:
                res = oracle.greedy_accept(*args, np.array([pos], np.int32))
            else:
                res = oracle.greedy_accept_stop(*args, list(stop_ids), np.array([n_new - len(out)], np.int32),
                                                np.array([pos], np.int32))
            n = int(res["n_emit"][0])
            out.extend(int(t) for t in res["emit"][0, :n])
            accepted_hist.append(int(res["accept_len"][0]))
            pos = int(res["pos_out"][0])
            x0 = int(res["next_tok"][0])
            if stop_ids is not None and res["done"][0]:
                break
        return out[:n_new], accepted_hist

    def generate_tree(self, prompt, n_new, drafter, stop_ids=None):
        """Tree drafts (DSSD fast.py _tree_cycle / _star_cycle): ``drafter(out)`` returns
        (parent, tokens) for the nodes below the root in creation order; one verify of
        the whole tree -> tree acceptance walk -> compaction of the accepted path's KV
        -> pos += a + 1. With stop_ids, the walk's outputs are truncated at the first
        stop token and at the tokens still allowed (DSSD _commit), the compaction moves
        only the committed nodes, and generation ends when the round says so."""
        self.reset()
        for i, x in enumerate(prompt[:-1]):
            self.forward_rows([x], i)
        x0, pos = prompt[-1], len(prompt) - 1
        out, accepted_hist = [], []
        while len(out) < n_new:
            par, toks = drafter(out)
            k = len(toks)
            parent = np.array([-1] + list(par), np.int32)
            g = self.forward_rows([x0] + [int(t) for t in toks], pos, parent=parent)
            res = oracle.tree_accept(g, np.array([toks], np.int32), k, np.array([k], np.int32), parent[None, :],
                                     None, 0, self.V, 1, k + 1, np.array([pos], np.int32))
            assert res["status"][0] == 0
            if stop_ids is not None:
                res = oracle.truncate_stop(res, k, list(stop_ids), np.array([n_new - len(out)], np.int32),
                                           np.array([pos], np.int32), path=res["path"])
            oracle.kv_compact(self.k_pool, self.v_pool, self.page_table, self.max_pages, np.array([pos], np.int32),
                              res["path"], res["accept_len"], k, res["status"], 1, self.Hkv, self.D)
            n = int(res["n_emit"][0])
            out.extend(int(t) for t in res["emit"][0, :n])
            accepted_hist.append(int(res["accept_len"][0]))
            pos = int(res["pos_out"][0])
            x0 = int(res["next_tok"][0])
            if stop_ids is not None and res["done"][0]:
                break
        return out[:n_new], accepted_hist
