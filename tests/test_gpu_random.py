"""Seeded random shapes against the oracle, beside the hand-picked cases: head dims,
query/kv head ratios, batch sizes, ragged k, positions from 0 up, split sizes and kmax
above the largest k for the chain and tree attention (tree shapes trie, star, random
and chain), and row / vocabulary / hidden sizes for the lm_head. Each case prints its
parameters first; the same tolerance as the other parity tests."""
import math

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import (assert_close, bits, check_argmax, gpu_attn, gpu_attn_tree, gpu_lm_head, oracle_attn,
                           oracle_attn_tree)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SPLITS = [0, 64, 128, 192, 256, 320, 512, 1024, 2048]


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _random_workload(seed, k_cap):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 6))
    k_lo = int(rng.integers(0, k_cap // 2 + 1))
    k_hi = int(rng.integers(k_lo, k_cap + 1))
    ctx_lo = int(rng.integers(0, 1500))
    ctx_hi = ctx_lo + int(rng.integers(0, 700))
    wl = synth.VerifyWorkload(f"rand{seed}", B=B, k=None, k_lo=k_lo, k_hi=k_hi, ctx_lo=ctx_lo, ctx_hi=ctx_hi,
                              Hq=G * Hkv, Hkv=Hkv, D=D, H=256, V=1000, max_pages=16, w_std=1 / 16)
    split = int(rng.choice(SPLITS))
    kmax = min(127, k_hi + int(rng.integers(0, 12)))
    return wl, split, kmax, rng


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_shapes(dev, seed):
    wl, split, kmax, _ = _random_workload(seed, 12)
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    print(f"[rand attn] seed {seed}: D={wl.D} Hq={wl.Hq} Hkv={wl.Hkv} B={len(x.pos)} pos {x.pos.tolist()} "
          f"k {x.k.tolist()} kmax {kmax} split {split}", flush=True)
    out, kp, vp, st = gpu_attn(x, dev, kv_split_tokens=split, kmax=kmax)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn(x)
    assert list(st) == list(st_ref) == [0] * len(x.pos)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, f"random attention seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_tree_attention_random_shapes(dev, seed):
    wl, split, _, rng = _random_workload(100 + seed, 20)
    shape = ["trie", "star", "random", "chain"][seed % 4]
    x = synth.make_verify_inputs(wl, seed=seed, with_lm_head=False)
    parent = synth.make_parents(x.k, seed, wl.name, shape, kmax=wl.kmax)
    print(f"[rand tree] seed {seed}: D={wl.D} Hq={wl.Hq} Hkv={wl.Hkv} B={len(x.pos)} pos {x.pos.tolist()} "
          f"k {x.k.tolist()} shape {shape} split {split}", flush=True)
    out, kp, vp, st = gpu_attn_tree(x, parent, dev, kv_split_tokens=split)
    rows, ref, kp_ref, vp_ref, st_ref = oracle_attn_tree(x, parent)
    assert (st == 0).all() and (st_ref == 0).all()
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy(), ref, f"random tree attention seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_lm_head_random_shapes(dev, seed):
    rng = np.random.default_rng(8000 + seed)
    R = int(rng.integers(1, 400))
    H = int(rng.choice([256, 512, 768, 1024]))
    V = int(rng.integers(1, 6000))
    print(f"[rand lm_head] seed {seed}: R={R} H={H} V={V}", flush=True)
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    g, mv = gpu_lm_head(h, w, dev)
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(h), bits(w), R, H, V)
    n_undecided = check_argmax(g, mv, g_ref, t1, t2, f"random lm_head seed {seed}")
    assert n_undecided <= max(2, R // 3)
