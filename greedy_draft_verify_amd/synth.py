"""Seeded synthetic workloads for the verify step.

This module only draws inputs: shapes, value distributions, page tables, draft
corruption. It holds none of the verify step's arithmetic, so both the HIP path
and the CPU oracle may take their inputs from it.

Every tensor gets its own seed, derived from ``(seed, workload, tensor)`` with
numpy's ``SeedSequence``; floating-point tensors are drawn in fp32 with a torch
generator on the requested device and rounded to bf16 (round-to-nearest-even).
Integer draws (positions, draft depths, corruption) use numpy's PCG64.

Workloads (names used by tests and the benchmark):

* ``tiny``    B=1, k=3, context 256, 4 q heads / 1 kv head, head_dim 64,
              32-page pool in a random permutation, hidden 256, vocab 1024.
* ``b16k4``   B=16, k=4, context U{512..4096}, 32q/8kv, head_dim 128, hidden 4096,
              vocab 151936, drafts corrupted with p=0.3.
* ``ragged``  B=64, k_s U{1..6}, context U{1024..32768}, 32q/8kv, head_dim 128,
              corruption p_s ~ U(0.2, 0.6) per sequence, every 8th sequence
              "first-seen" (all-random drafts).
* ``long``    B=8, k=6, context 131072, 16q/2kv, head_dim 256, hidden 5120,
              vocab 151936, 32768-entry draft->target id map.
* ``delta``   Gated DeltaNet: B=32, T=5, 32 heads, d_k=d_v=128.
* ``b16tree`` the b16k4 shapes with a 16-node draft tree per sequence (k=15):
              a spine of head drafts created first, then side branches (trie) or
              star siblings at the root; see ``make_parents``.

The pool holds every page of every sequence plus a quarter spare, shuffled; the
pages a sequence does not own are random bf16 too, so any leak into a result
shows. Page-table entries past a sequence's last needed page are -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 16


@dataclass(frozen=True)
class VerifyWorkload:
    name: str
    B: int
    k: int | None               # uniform draft depth, or None for k_s ~ U{k_lo..k_hi}
    k_lo: int
    k_hi: int
    ctx_lo: int
    ctx_hi: int
    Hq: int
    Hkv: int
    D: int
    H: int
    V: int
    max_pages: int              # page-table width (the sequences' capacity)
    p_corrupt: tuple = (0.3, 0.3)   # per-sequence corruption prob ~ U(lo, hi)
    first_seen_every: int = 0   # every n-th sequence (s % n == n-1) gets random drafts
    n_d2t: int = 0              # trimmed draft vocabulary size (0: none)
    pool_pages: int = 0         # 0: 1.25 x pages needed
    w_std: float = field(default=0.0)

    @property
    def kmax(self) -> int:
        return self.k if self.k is not None else self.k_hi


WORKLOADS = {
    "tiny": VerifyWorkload("tiny", B=1, k=3, k_lo=3, k_hi=3, ctx_lo=256, ctx_hi=256, Hq=4, Hkv=1,
                           D=64, H=256, V=1024, max_pages=32, pool_pages=32, w_std=1 / 16),
    "b16k4": VerifyWorkload("b16k4", B=16, k=4, k_lo=4, k_hi=4, ctx_lo=512, ctx_hi=4096, Hq=32,
                            Hkv=8, D=128, H=4096, V=151936, max_pages=(4096 + 64) // PAGE,
                            w_std=1 / 64),
    "ragged": VerifyWorkload("ragged", B=64, k=None, k_lo=1, k_hi=6, ctx_lo=1024, ctx_hi=32768,
                             Hq=32, Hkv=8, D=128, H=4096, V=151936,
                             max_pages=(32768 + 64) // PAGE, p_corrupt=(0.2, 0.6),
                             first_seen_every=8, w_std=1 / 64),
    "long": VerifyWorkload("long", B=8, k=6, k_lo=6, k_hi=6, ctx_lo=131072, ctx_hi=131072, Hq=16,
                           Hkv=2, D=256, H=5120, V=151936, max_pages=(131072 + 64) // PAGE,
                           n_d2t=32768, w_std=1 / math.sqrt(5120)),
}

WORKLOADS["b16tree"] = VerifyWorkload("b16tree", B=16, k=15, k_lo=15, k_hi=15, ctx_lo=512, ctx_hi=4096,
                                      Hq=32, Hkv=8, D=128, H=4096, V=151936,
                                      max_pages=(4096 + 64) // PAGE, w_std=1 / 64)

TENSOR_IDS = {name: i for i, name in enumerate(
    ["pos", "k", "pool_perm", "k_pool", "v_pool", "q", "k_new", "v_new", "hidden", "w", "drafts",
     "corrupt", "d2t", "dq", "dk", "dv", "da", "db", "dstate", "dL", "extra", "parent"])}
WORKLOAD_IDS = {"tiny": 1, "b16k4": 2, "ragged": 3, "long": 4, "delta": 5, "b16tree": 6}


def tensor_seed(seed: int, workload: str, tensor: str) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(WORKLOAD_IDS.get(workload, 99), TENSOR_IDS[tensor]))
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def np_rng(seed: int, workload: str, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(tensor_seed(seed, workload, tensor)))


def torch_gen(seed: int, workload: str, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, workload, tensor))
    return g


def normal_bf16(shape, std, seed, workload, tensor, device="cpu", slab=1 << 26) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded to bf16; drawn in slabs to bound fp32 temporaries."""
    g = torch_gen(seed, workload, tensor, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for i in range(0, n, slab):
        m = min(slab, n - i)
        x = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[i:i + m].copy_(x)
    return out


def pages_needed(pos: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Pages covering positions 0 .. pos + k (the rows' own slots included)."""
    return (pos + k) // PAGE + 1


@dataclass
class VerifyInputs:
    wl: VerifyWorkload
    pos: np.ndarray            # [B] int32, tokens already cached = position of row 0
    k: np.ndarray              # [B] int32
    R: int
    page_table: np.ndarray     # [B, max_pages] int32
    n_pages: int
    q: torch.Tensor            # [R, Hq, D] bf16
    k_new: torch.Tensor        # [R, Hkv, D] bf16
    v_new: torch.Tensor        # [R, Hkv, D] bf16
    k_pool: torch.Tensor       # [n_pages, Hkv, 16 * D] bf16 (pool block layout)
    v_pool: torch.Tensor       # [n_pages, Hkv, 16 * D] bf16 (pool block layout)
    hidden: torch.Tensor       # [R, H] bf16
    w: torch.Tensor            # [V, H] bf16
    d2t: np.ndarray | None     # [n_d2t] int32

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.wl.D)


def make_verify_inputs(name, seed: int = 0, device="cpu", with_lm_head: bool = True,
                       B: int | None = None, ctx: int | None = None) -> VerifyInputs:
    """Draw one verify batch for a named workload (or a VerifyWorkload). ``B`` / ``ctx``
    override the batch size and context (smaller instances of the same shape)."""
    wl = WORKLOADS[name] if isinstance(name, str) else name
    name = wl.name
    Bn = wl.B if B is None else B
    rng_pos = np_rng(seed, name, "pos")
    if ctx is not None:
        pos = np.full(Bn, ctx, np.int32)
    else:
        pos = rng_pos.integers(wl.ctx_lo, wl.ctx_hi + 1, size=Bn).astype(np.int32)
    if wl.k is not None:
        k = np.full(Bn, wl.k, np.int32)
    else:
        k = np_rng(seed, name, "k").integers(wl.k_lo, wl.k_hi + 1, size=Bn).astype(np.int32)
    R = int((k + 1).sum())
    need = pages_needed(pos.astype(np.int64), k.astype(np.int64))
    max_pages = max(wl.max_pages, int(need.max()))
    total = int(need.sum())
    n_pages = wl.pool_pages if (wl.pool_pages and wl.pool_pages >= total) else int(math.ceil(total * 1.25))
    perm = np_rng(seed, name, "pool_perm").permutation(n_pages).astype(np.int32)
    page_table = np.full((Bn, max_pages), -1, np.int32)
    cur = 0
    for s in range(Bn):
        page_table[s, :need[s]] = perm[cur:cur + need[s]]
        cur += int(need[s])
    k_pool = normal_bf16((n_pages, wl.Hkv, PAGE * wl.D), 1.0, seed, name, "k_pool", device)
    v_pool = normal_bf16((n_pages, wl.Hkv, PAGE * wl.D), 1.0, seed, name, "v_pool", device)
    q = normal_bf16((R, wl.Hq, wl.D), 1.0, seed, name, "q", device)
    k_new = normal_bf16((R, wl.Hkv, wl.D), 1.0, seed, name, "k_new", device)
    v_new = normal_bf16((R, wl.Hkv, wl.D), 1.0, seed, name, "v_new", device)
    if with_lm_head:
        hidden = normal_bf16((R, wl.H), 1.0, seed, name, "hidden", device)
        w = normal_bf16((wl.V, wl.H), wl.w_std, seed, name, "w", device)
    else:
        hidden = torch.empty((0, wl.H), dtype=torch.bfloat16, device=device)
        w = torch.empty((0, wl.H), dtype=torch.bfloat16, device=device)
    d2t = None
    if wl.n_d2t:
        d2t = np_rng(seed, name, "d2t").permutation(wl.V)[:wl.n_d2t].astype(np.int32)
    return VerifyInputs(wl, pos, k, R, page_table, n_pages, q, k_new, v_new, k_pool, v_pool,
                        hidden, w, d2t)


def make_drafts(wl: VerifyWorkload, k: np.ndarray, true_next: np.ndarray, seed: int = 0,
                d2t: np.ndarray | None = None) -> np.ndarray:
    """Drafts [B, kmax] int32 from the target's greedy tokens.

    ``true_next[s][j]`` (j < k_s) is the token the target would emit after row j of
    sequence s, i.e. the greedy token of that verify row. Each draft starts as that
    token and, with the sequence's corruption probability, is replaced by a uniform
    id different from it. First-seen sequences get uniform drafts. With a d2t map,
    drafts are draft-vocabulary ids: the true token's draft id when the map holds
    it, otherwise a random draft id (which then cannot match). Unused slots are -1.
    """
    B = len(k)
    kmax = wl.kmax
    rc = np_rng(seed, wl.name, "corrupt")
    rd = np_rng(seed, wl.name, "drafts")
    space = wl.n_d2t if d2t is not None else wl.V
    inv = None
    if d2t is not None:
        inv = {int(t): i for i, t in enumerate(d2t)}
    p_lo, p_hi = wl.p_corrupt
    drafts = np.full((B, max(kmax, 1)), -1, np.int32)
    for s in range(B):
        p = rc.uniform(p_lo, p_hi)
        first_seen = wl.first_seen_every and (s % wl.first_seen_every == wl.first_seen_every - 1)
        for j in range(int(k[s])):
            if first_seen:
                drafts[s, j] = rd.integers(0, space)
                continue
            t = int(true_next[s][j])
            if inv is not None:
                truth = inv.get(t, -1)
                if truth < 0:
                    drafts[s, j] = rd.integers(0, space)
                    continue
            else:
                truth = t
            if rc.uniform() < p:
                x = int(rd.integers(0, space - 1))
                drafts[s, j] = x + (x >= truth)
            else:
                drafts[s, j] = truth
    return drafts


def make_parents(k: np.ndarray, seed: int = 0, name: str = "b16tree", shape: str = "trie",
                 kmax: int | None = None, spine_frac: float = 0.5) -> np.ndarray:
    """Parent lists [B, kmax + 1] int32 of draft trees in creation order (node 0 = root,
    parent -1; node i's parent in [0, i)); entries past k_s are -1.

    shape "chain": parent i - 1. "star": every node a child of the root (depth 1).
    "trie": like a tree draft grown by a head chain and then widened: the first
    round(spine_frac * k_s) nodes form a spine under the root, each later node hangs
    under a uniformly drawn earlier node (spine nodes twice as likely).
    "random": every node under a uniformly drawn earlier node.
    """
    B = len(k)
    kmax = int(np.max(k)) if kmax is None else kmax
    rng = np_rng(seed, name, "parent")
    par = np.full((B, kmax + 1), -1, np.int32)
    for s in range(B):
        ks = int(k[s])
        n_spine = int(round(spine_frac * ks))
        for i in range(1, ks + 1):
            if shape == "chain":
                par[s, i] = i - 1
            elif shape == "star":
                par[s, i] = 0
            elif shape == "random":
                par[s, i] = int(rng.integers(0, i))
            elif shape == "trie":
                if i <= n_spine:
                    par[s, i] = i - 1
                else:
                    w = np.array([2.0 if j <= n_spine else 1.0 for j in range(i)])
                    par[s, i] = int(rng.choice(i, p=w / w.sum()))
            else:
                raise ValueError(shape)
    return par


def make_tree_drafts(wl: VerifyWorkload, k: np.ndarray, parent: np.ndarray, target: np.ndarray,
                     seed: int = 0) -> np.ndarray:
    """Drafts [B, kmax] int32 for tree nodes from the target's greedy tokens.

    ``target[s][u]`` is the greedy token of node u's row. Node i's draft starts as the
    target of its parent (the token that would be accepted there) and, with the
    sequence's corruption probability, is replaced by a uniform id different from it.
    Unused slots are -1.
    """
    B = len(k)
    kmax = parent.shape[1] - 1
    rc = np_rng(seed, wl.name, "corrupt")
    rd = np_rng(seed, wl.name, "drafts")
    p_lo, p_hi = wl.p_corrupt
    drafts = np.full((B, max(kmax, 1)), -1, np.int32)
    for s in range(B):
        p = rc.uniform(p_lo, p_hi)
        for i in range(1, int(k[s]) + 1):
            truth = int(target[s][parent[s, i]])
            if rc.uniform() < p:
                x = int(rd.integers(0, wl.V - 1))
                drafts[s, i - 1] = x + (x >= truth)
            else:
                drafts[s, i - 1] = truth
    return drafts


@dataclass
class DeltaInputs:
    B: int
    T: int
    Hd: int
    dk: int
    dv: int
    q: torch.Tensor       # [B, T, Hd, dk] bf16
    k: torch.Tensor       # [B, T, Hd, dk] bf16, L2-normalised before rounding
    v: torch.Tensor       # [B, T, Hd, dv] bf16
    a: torch.Tensor       # [B, T, Hd] fp32 ~ U(0.9, 1)
    b: torch.Tensor       # [B, T, Hd] fp32 ~ U(0, 1)
    state: torch.Tensor   # [B, Hd, dv, dk] fp32 ~ N(0, 1/128)
    L: np.ndarray         # [B] int32 ~ U{0..T}


def make_delta_inputs(seed: int = 0, device="cpu", B=32, T=5, Hd=32, dk=128, dv=128) -> DeltaInputs:
    name = "delta"
    q = normal_bf16((B, T, Hd, dk), 1.0, seed, name, "dq", device)
    g = torch_gen(seed, name, "dk", device)
    kf = torch.randn((B, T, Hd, dk), generator=g, device=device, dtype=torch.float32)
    kf = kf / kf.norm(dim=-1, keepdim=True)
    k = kf.to(torch.bfloat16)
    v = normal_bf16((B, T, Hd, dv), 1.0, seed, name, "dv", device)
    a = 0.9 + 0.1 * torch.rand((B, T, Hd), generator=torch_gen(seed, name, "da", device),
                               device=device, dtype=torch.float32)
    b = torch.rand((B, T, Hd), generator=torch_gen(seed, name, "db", device), device=device,
                   dtype=torch.float32)
    state = torch.randn((B, Hd, dv, dk), generator=torch_gen(seed, name, "dstate", device),
                        device=device, dtype=torch.float32) * math.sqrt(1.0 / 128)
    L = np_rng(seed, name, "dL").integers(0, T + 1, size=B).astype(np.int32)
    return DeltaInputs(B, T, Hd, dk, dv, q, k, v, a, b, state, L)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 tensor as a host uint16 array."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
