"""Lossless invariant on the GPU: greedy speculative decoding through the library
emits exactly the stream that one-row greedy decoding through the same library
emits (span-02 spec.rs module doc; DSSD fast.py generate_ar as the reference stream).

A toy one-layer model (tiny-workload sizes: vocabulary 1024, hidden 256, 4 q heads
/ 1 kv head, head_dim 64) whose attention, lm_head + argmax and acceptance run in
the HIP kernels; the projections between them are glue computed on the host one
row at a time in fp64, so a row's glue never depends on how many rows share a step.
Because the kernels are row-invariant, a verify row is bit-identical to the
one-row step at the same position and the two streams must match token for token.
"""
import math

import numpy as np
import pytest
import torch

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

V, H, HQ, HKV, D = 1024, 256, 4, 1, 64
N_NEW = 64


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


class GpuToy:
    def __init__(self, dev, seed=0, max_pages=64):
        import greedy_draft_verify_amd as gdv
        self.gdv = gdv
        rng = np.random.default_rng(seed)
        r = lambda *s: rng.standard_normal(s)
        self.E = bf16(r(V, H)).double().numpy()
        self.Wq = bf16(r(HQ * D, H) / 16).double().numpy()
        self.Wk = bf16(r(HKV * D, H) / 16).double().numpy()
        self.Wv = bf16(r(HKV * D, H) / 16).double().numpy()
        self.Wo = bf16(r(H, HQ * D) / 16).double().numpy()
        self.dev = dev
        wlm = bf16(r(V, H) / 16)
        self.Wlm = wlm.double().numpy()
        self.wp = gdv.spec_lm_head_pack(wlm.to(dev))
        self.max_pages = max_pages
        self.n_pages = 2 * max_pages
        self.pt = torch.from_numpy(rng.permutation(self.n_pages)[:max_pages].astype(np.int32)[None, :]).to(dev)

    def reset(self):
        self.kp = torch.zeros((self.n_pages, HKV, 16 * D), dtype=torch.bfloat16, device=self.dev)
        self.vp = torch.zeros_like(self.kp)

    def rows(self, tokens, pos, kmax, parent=None, gaps=None):
        """Attention + lm_head for rows tokens[j] at positions pos + j (or the nodes of a
        draft tree with parent list ``parent`` [kmax + 1]); greedy tokens. With ``gaps``
        (a list), appends each row's top-2 logit gap, computed on the host in fp64."""
        gdv, dev = self.gdv, self.dev
        T = len(tokens)
        e = self.E[tokens]                                               # [T, H] fp64 (exact bf16 values)
        proj = lambda W: bf16(np.stack([W @ e[j] for j in range(T)]))   # one row at a time
        q = proj(self.Wq).view(T, HQ, D).to(dev)
        kn = proj(self.Wk).view(T, HKV, D).to(dev)
        vn = proj(self.Wv).view(T, HKV, D).to(dev)
        out = torch.empty((T, HQ, D), dtype=torch.bfloat16, device=dev)
        st = torch.empty(1, dtype=torch.int32, device=dev)
        i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
        if parent is None:
            gdv.spec_verify_attn(q, kn, vn, self.kp, self.vp, self.pt, i32([pos]), i32([T - 1]), kmax,
                                 1 / math.sqrt(D), out, st)
        else:
            gdv.spec_verify_attn_tree(q, kn, vn, self.kp, self.vp, self.pt, i32([pos]), i32([T - 1]),
                                      i32([list(parent)]), 1 / math.sqrt(D), out, st)
        att = out.double().cpu().numpy().reshape(T, HQ * D)
        hb = bf16(np.stack([e[j] + self.Wo @ att[j] for j in range(T)]))
        if gaps is not None:
            for j in range(T):
                top = np.sort(self.Wlm @ hb[j].double().numpy())
                gaps.append(float(top[-1] - top[-2]))
        h = hb.to(dev)
        am = torch.empty(T, dtype=torch.int32, device=dev)
        gdv.spec_lm_head_argmax(h, self.wp, V, am)
        torch.cuda.synchronize()
        assert st.item() == 0
        return am.cpu().numpy()

    def generate_ar(self, prompt, n, kmax, gaps=None):
        """One-row greedy decoding; ``gaps`` (a list) receives, for every emitted token,
        the top-2 logit gap of the row that chose it."""
        self.reset()
        g = None
        for i, t in enumerate(prompt):
            gl = []
            g = int(self.rows([t], i, kmax, gaps=gl)[0])
        out, pos = [], len(prompt)
        while len(out) < n:
            out.append(g)
            if gaps is not None:
                gaps.append(gl[0])
            gl = []
            g = int(self.rows([g], pos, kmax, gaps=gl)[0])
            pos += 1
        return out

    def generate_tree(self, prompt, n, drafter, kmax, stop_ids=None):
        """Tree drafts: ``drafter(out)`` gives (parents, tokens) of the nodes below the root in
        creation order; one tree verify, the acceptance walk, compaction, pos += a + 1.
        With stop_ids, the walk's outputs are truncated on the device (stop tokens and the
        tokens still allowed) before compaction, and generation ends when a round says so."""
        gdv, dev = self.gdv, self.dev
        self.reset()
        for i, t in enumerate(prompt[:-1]):
            self.rows([t], i, kmax)
        x0, pos = prompt[-1], len(prompt) - 1
        out, hist = [], []
        i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
        while len(out) < n:
            par, toks = drafter(out)
            k = len(toks)
            parent = [-1] + list(par) + [-1] * (kmax - k)
            drafts = [int(t) for t in toks] + [-1] * (kmax - k)
            g = self.rows([x0] + [int(t) for t in toks], pos, kmax, parent=parent)
            z = lambda: torch.empty(1, dtype=torch.int32, device=dev)
            pos_out, acc, ne, nt, st = z(), z(), z(), z(), z()
            emit = torch.empty((1, kmax + 1), dtype=torch.int32, device=dev)
            path = torch.empty((1, kmax), dtype=torch.int32, device=dev)
            pos_t = i32([pos])
            gdv.spec_tree_accept(i32(g), i32([drafts]), i32([k]), i32([parent]), None, V, pos_t, pos_out, acc, ne,
                                 emit, nt, path, st)
            done = torch.zeros(1, dtype=torch.int32, device=dev)
            if stop_ids is not None:
                gdv.spec_truncate_stop(i32(list(stop_ids)), i32([n - len(out)]), pos_t, pos_out, acc, ne, emit, nt,
                                       done, st, path=path)
            gdv.spec_kv_compact(self.kp, self.vp, self.pt, pos_t, path, acc, st)
            torch.cuda.synchronize()
            assert st.item() == 0
            m = ne.item()
            out.extend(emit.cpu().numpy()[0, :m].tolist())
            hist.append(acc.item())
            pos, x0 = pos_out.item(), nt.item()
            if done.item():
                break
        return out[:n], hist

    def generate_spec(self, prompt, n, drafter, k):
        gdv, dev = self.gdv, self.dev
        self.reset()
        for i, t in enumerate(prompt[:-1]):
            self.rows([t], i, k)
        x0, pos = prompt[-1], len(prompt) - 1
        out, hist = [], []
        i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
        while len(out) < n:
            drafts = [int(d) for d in drafter(out, k)]
            g = self.rows([x0] + drafts, pos, k)
            z = lambda: torch.empty(1, dtype=torch.int32, device=dev)
            pos_out, acc, ne, nt, st = z(), z(), z(), z(), z()
            emit = torch.empty((1, k + 1), dtype=torch.int32, device=dev)
            gdv.spec_greedy_accept(i32(g), i32([drafts]), i32([k]), None, V, i32([pos]), pos_out, acc, ne, emit, nt, st)
            torch.cuda.synchronize()
            m = ne.item()
            out.extend(emit.cpu().numpy()[0, :m].tolist())
            hist.append(acc.item())
            pos, x0 = pos_out.item(), nt.item()
        return out[:n], hist


@pytest.fixture(scope="module")
def toy():
    dev = torch.device("cuda:0")
    m = GpuToy(dev)
    prompt = list(np.random.default_rng(1).integers(0, V, 24))
    ref = m.generate_ar(prompt, N_NEW + 8, kmax=6)
    return m, prompt, ref


@pytest.fixture(scope="module")
def toy_tree():
    dev = torch.device("cuda:0")
    m = GpuToy(dev)
    prompt = list(np.random.default_rng(1).integers(0, V, 24))
    gaps = []
    ref = m.generate_ar(prompt, N_NEW + 16, kmax=15, gaps=gaps)
    return m, prompt, ref, gaps


@pytest.mark.parametrize("kind,k", [("perfect", 4), ("corrupt", 4), ("random", 3), ("corrupt", 6)])
def test_gpu_spec_stream_equals_one_row_stream(toy, kind, k):
    m, prompt, ref = toy
    rng = np.random.default_rng(11)

    def drafter(out, kk):
        true = ref[len(out):len(out) + kk]
        true = true + [0] * (kk - len(true))
        if kind == "perfect":
            return true
        if kind == "random":
            return list(rng.integers(0, V, kk))
        return [t if rng.uniform() >= 0.3 else int((t + 1 + rng.integers(0, V - 1)) % V) for t in true]

    out, hist = m.generate_spec(prompt, N_NEW, drafter, k)
    assert out == ref[:N_NEW]
    if kind == "perfect":
        assert min(hist[:-1]) == k


@pytest.mark.parametrize("shape", ["star", "spine", "trie", "random"])
def test_gpu_tree_stream_equals_one_row_stream(toy_tree, shape):
    """Tree cycles (attention over tree rows, the acceptance walk, compaction) emit the
    one-row stream token for token, whatever the tree's shape: every tree row is the
    bytes of its one-row decode after compaction."""
    m, prompt, ref, gaps = toy_tree
    rng = np.random.default_rng(12)

    def drafter(out):
        true = ref[len(out):len(out) + 8]
        true = true + [0] * (8 - len(true))
        wrong = lambda t: int((t + 1 + rng.integers(0, V - 1)) % V)
        if shape == "star":
            kids = [wrong(true[0]) for _ in range(4)]
            if rng.uniform() < 0.8:
                kids[int(rng.integers(0, 4))] = true[0]
            return [0] * 4, kids
        if shape == "random":     # each node under a uniformly drawn earlier node
            par, toks, depth = [], [], [0]
            for _ in range(12):
                p = int(rng.integers(0, len(toks) + 1))
                p = p if depth[p] < 7 else 0
                d = depth[p]
                par.append(p)
                toks.append(true[d] if rng.uniform() < 0.7 else wrong(true[d]))
                depth.append(d + 1)
            return par, toks
        par, toks, spine = [], [], [0]
        for d in range(6):
            par.append(spine[-1])
            toks.append(true[d] if rng.uniform() < 0.8 else wrong(true[d]))
            spine.append(len(toks))
        if shape == "trie":       # side branches created after the spine, some holding the truth
            for d in range(6):
                if rng.uniform() < 0.6:
                    par.append(spine[d])
                    toks.append(true[d] if toks[spine[d + 1] - 1] != true[d] else wrong(true[d]))
        return par, toks

    out, hist = m.generate_tree(prompt, N_NEW, drafter, kmax=15)
    n_same = next((i for i, (a, b) in enumerate(zip(out, ref)) if a != b), N_NEW)
    assert n_same == N_NEW, (n_same, gaps[n_same])
    assert max(hist) >= (3 if shape in ("spine", "trie") else 1)


@pytest.mark.parametrize("limit", [False, True])
def test_gpu_tree_stream_with_stop_ends_where_one_row_decoding_ends(toy_tree, limit):
    """Spine-shaped trees (exact bytes) with a stop token, truncated on the device:
    the stream is the one-row stream up to and including the stop token's first
    appearance; with only a limit, it is the first n tokens exactly."""
    m, prompt, ref, _ = toy_tree
    rng = np.random.default_rng(13)

    def drafter(out):
        true = ref[len(out):len(out) + 8]
        true = true + [0] * (8 - len(true))
        par, toks = [], []
        for d in range(6):
            par.append(d)
            toks.append(true[d] if rng.uniform() < 0.8 else int((true[d] + 1 + rng.integers(0, V - 1)) % V))
        return par, toks

    if limit:
        n = N_NEW - 7
        out, _ = m.generate_tree(prompt, n, drafter, kmax=15, stop_ids=())
        assert out == ref[:n]
    else:
        stop = ref[N_NEW // 2]
        want = ref[:ref.index(stop) + 1]
        out, _ = m.generate_tree(prompt, N_NEW, drafter, kmax=15, stop_ids=(stop,))
        assert out == want

