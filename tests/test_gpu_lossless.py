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
        self.wp = gdv.spec_lm_head_pack(bf16(r(V, H) / 16).to(dev))
        self.max_pages = max_pages
        self.n_pages = 2 * max_pages
        self.pt = torch.from_numpy(rng.permutation(self.n_pages)[:max_pages].astype(np.int32)[None, :]).to(dev)

    def reset(self):
        self.kp = torch.zeros((self.n_pages, HKV, 16 * D), dtype=torch.bfloat16, device=self.dev)
        self.vp = torch.zeros_like(self.kp)

    def rows(self, tokens, pos, kmax):
        """Attention + lm_head for rows tokens[j] at positions pos + j; greedy tokens."""
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
        gdv.spec_verify_attn(q, kn, vn, self.kp, self.vp, self.pt, i32([pos]), i32([T - 1]), kmax, 1 / math.sqrt(D),
                             out, st)
        att = out.double().cpu().numpy().reshape(T, HQ * D)
        h = bf16(np.stack([e[j] + self.Wo @ att[j] for j in range(T)])).to(dev)
        am = torch.empty(T, dtype=torch.int32, device=dev)
        gdv.spec_lm_head_argmax(h, self.wp, V, am)
        torch.cuda.synchronize()
        assert st.item() == 0
        return am.cpu().numpy()

    def generate_ar(self, prompt, n, kmax):
        self.reset()
        g = None
        for i, t in enumerate(prompt):
            g = int(self.rows([t], i, kmax)[0])
        out, pos = [], len(prompt)
        while len(out) < n:
            out.append(g)
            g = int(self.rows([g], pos, kmax)[0])
            pos += 1
        return out

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
