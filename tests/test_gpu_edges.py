"""Edge cases of the verify path on the GPU, against the oracle.

* attention at the position edges: an empty cache (pos = 0, the row attends only to
  its own appended key), rows straddling a page boundary and a split boundary, and
  rows ending in the last slot the page table covers; default and 64-token splits;
* the largest batch the attention accepts (B = 4096 sequences, k_s in 0..2, contexts
  0..40 including empty ones), every row checked;
* the lm_head with many row groups (640 and 1000 rows: 5 and 8 groups of 16-row tiles).
Tolerance as in the other parity tests: |err| <= 2e-2 + 1e-2 |ref|; append bit-exact.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available
from tests.helpers import assert_close, bits, check_argmax, gpu_attn, gpu_lm_head, oracle_attn

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _wl(name, B, k_lo, k_hi, ctx_lo, ctx_hi, Hq, Hkv, D, max_pages, H=256, V=1000):
    return synth.VerifyWorkload(name, B=B, k=None, k_lo=k_lo, k_hi=k_hi, ctx_lo=ctx_lo, ctx_hi=ctx_hi, Hq=Hq,
                                Hkv=Hkv, D=D, H=H, V=V, max_pages=max_pages, w_std=1 / math.sqrt(H))


@pytest.mark.parametrize("split", [0, 64])
def test_attention_position_edges(dev, split):
    # every sequence owns all 16 table entries (pos 252 + k 3 reaches slot 255)
    wl = _wl("edges", 6, 3, 3, 252, 252, 8, 2, 128, 16)
    x = synth.make_verify_inputs(wl, seed=9, with_lm_head=False)
    assert x.page_table.shape[1] == 16 and (x.page_table >= 0).all()
    pos = np.array([0, 0, 15, 63, 64, 252], np.int32)
    k = np.array([0, 3, 1, 2, 3, 3], np.int32)
    R = int((k + 1).sum())
    y = dataclasses.replace(x, pos=pos, k=k, R=R, q=x.q[:R], k_new=x.k_new[:R], v_new=x.v_new[:R])
    out, kp, vp, st = gpu_attn(y, dev, kv_split_tokens=split, kmax=3)
    assert (st == 0).all()
    rows, ref, kp_ref, vp_ref, _ = oracle_attn(y)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy()[rows], ref, f"position edges (split {split})")
    # an empty cache and k = 0: the only key is the row's own, so the output is its V
    o0 = out.float().cpu().numpy()[0]
    v0 = x.v_new[0].float().cpu().numpy()                       # [Hkv, D]
    G = wl.Hq // wl.Hkv
    for h in range(wl.Hq):
        assert np.array_equal(o0[h], v0[h // G])


def test_attention_largest_batch(dev):
    wl = _wl("many", 4096, 0, 2, 0, 40, 2, 1, 64, 4)
    x = synth.make_verify_inputs(wl, seed=10, with_lm_head=False)
    assert (x.pos == 0).any()
    out, kp, vp, st = gpu_attn(x, dev)
    assert (st == 0).all()
    rows, ref, kp_ref, vp_ref, _ = oracle_attn(x)
    assert np.array_equal(bits(kp), kp_ref) and np.array_equal(bits(vp), vp_ref)
    assert_close(out.float().cpu().numpy()[rows], ref, "B=4096")


@pytest.mark.parametrize("R", [640, 1000])
def test_lm_head_many_row_groups(dev, R):
    H, V = 256, 300
    rng = np.random.default_rng(R)
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    g, mv = gpu_lm_head(h, w, dev)
    g_ref, t1, t2, _ = oracle.lm_head_argmax(bits(h), bits(w), R, H, V)
    n_und = check_argmax(g, mv, g_ref, t1, t2, f"lm_head R={R}")
    assert n_und <= R // 3
