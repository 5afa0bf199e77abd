"""Shared runners for the parity tests: the same seeded inputs go through the HIP
library (via the binding) and through the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from greedy_draft_verify_amd import synth

ATOL, RTOL = 2e-2, 1e-2      # attention / logits / DeltaNet tolerance (bf16 in, fp32 accumulate)
GAP = 5e-2                   # argmax must agree where the oracle's top-2 gap exceeds this

bits = synth.bf16_bits


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


def within_tol(got, ref, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    excess = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    return excess, bool((excess <= 0).all())


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    excess, ok = within_tol(got, ref, atol, rtol)
    if not ok:
        idx = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError(f"{what}: {int((excess > 0).sum())} of {excess.size} outside "
                             f"{atol} + {rtol}|ref|; worst at {idx}: got {np.asarray(got)[idx]} "
                             f"ref {np.asarray(ref)[idx]}")


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def gpu_attn(x: synth.VerifyInputs, dev, kv_split_tokens=0, pos=None, k=None, page_table=None,
             k_pool=None, v_pool=None, q=None, k_new=None, v_new=None, kmax=None):
    """Runs spec_verify_attn; returns (out bf16 [R,Hq,D] device, k_pool, v_pool, status np)."""
    pos = x.pos if pos is None else pos
    k = x.k if k is None else k
    pt = x.page_table if page_table is None else page_table
    q = x.q if q is None else q
    k_new = x.k_new if k_new is None else k_new
    v_new = x.v_new if v_new is None else v_new
    R = q.shape[0]
    kp = (x.k_pool if k_pool is None else k_pool).to(dev).clone()
    vp = (x.v_pool if v_pool is None else v_pool).to(dev).clone()
    out = torch.full((R, x.wl.Hq, x.wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    status = torch.full((len(pos),), -7, dtype=torch.int32, device=dev)
    import greedy_draft_verify_amd as gdv
    if kmax is None:
        kmax = max(int(np.max(k)), 0)
    gdv.spec_verify_attn(q.to(dev).contiguous(), k_new.to(dev).contiguous(), v_new.to(dev).contiguous(), kp,
                         vp, i32(pt, dev), i32(pos, dev), i32(k, dev), kmax, x.scale, out, status,
                         kv_split_tokens=kv_split_tokens)
    torch.cuda.synchronize()
    return out, kp, vp, status.cpu().numpy()


def oracle_attn(x: synth.VerifyInputs, seqs=None, k_pool_bits=None, v_pool_bits=None):
    """Oracle attention for the selected sequences (all by default).

    Returns (rows: global row indices [n], out fp64 [n,Hq,D], k_pool_after, v_pool_after, status)."""
    wl = x.wl
    B = len(x.pos)
    seqs = list(range(B)) if seqs is None else list(seqs)
    off_all = np.concatenate([[0], np.cumsum(x.k + 1)]).astype(np.int64)
    rows = np.concatenate([np.arange(off_all[s], off_all[s + 1]) for s in seqs])
    kp = (bits(x.k_pool) if k_pool_bits is None else k_pool_bits).copy()
    vp = (bits(x.v_pool) if v_pool_bits is None else v_pool_bits).copy()
    pos, k, pt = x.pos[seqs], x.k[seqs], x.page_table[seqs]
    qb, knb, vnb = bits(x.q)[rows], bits(x.k_new)[rows], bits(x.v_new)[rows]
    R = len(rows)
    off, st = oracle.validate(pt, pt.shape[1], x.n_pages, pos, k, -1, len(seqs), R)
    oracle.append_kv(knb, vnb, kp, vp, pt, pt.shape[1], pos, k, off, st, len(seqs), wl.Hkv, wl.D)
    out = oracle.verify_attn(qb, kp, vp, pt, pt.shape[1], pos, k, off, st, len(seqs), R, wl.Hq, wl.Hkv, wl.D,
                             x.scale)
    return rows, out, kp, vp, st


# ---------------------------------------------------------------------------
# lm_head
# ---------------------------------------------------------------------------
def gpu_lm_head(hidden, w, dev, w_packed=None):
    """Packs w (unless a packed copy is given) and runs spec_lm_head_argmax."""
    import greedy_draft_verify_amd as gdv
    R = hidden.shape[0]
    V = w.shape[0]
    if w_packed is None:
        w_packed = gdv.spec_lm_head_pack(w.to(dev).contiguous())
    am = torch.full((R,), -5, dtype=torch.int32, device=dev)
    mv = torch.full((R,), float("nan"), dtype=torch.float32, device=dev)
    gdv.spec_lm_head_argmax(hidden.to(dev).contiguous(), w_packed, V, am, mv)
    torch.cuda.synchronize()
    return am.cpu().numpy(), mv.cpu().numpy()


def check_argmax(g_gpu, mv_gpu, g_ref, top1, top2, what):
    """Argmax must agree where the oracle's top-2 gap > GAP; maxval within tolerance."""
    decided = (top1 - top2) > GAP
    bad = np.nonzero(decided & (g_gpu != g_ref))[0]
    assert len(bad) == 0, f"{what}: argmax differs at rows {bad[:10]} (gpu {g_gpu[bad[:10]]} ref {g_ref[bad[:10]]})"
    assert_close(mv_gpu, top1, f"{what} maxval")
    # an undecided row's GPU pick must still be a near-maximum
    return int((~decided).sum())


# ---------------------------------------------------------------------------
# accept
# ---------------------------------------------------------------------------
def gpu_accept(g, drafts, k, d2t, V, pos, dev, kmax=None):
    import greedy_draft_verify_amd as gdv
    B = len(k)
    drafts = np.ascontiguousarray(drafts, np.int32)
    kmax = drafts.shape[1] if kmax is None else kmax
    z = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = z(), z(), z(), z(), z()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    gdv.spec_greedy_accept(i32(g, dev), i32(drafts, dev), i32(k, dev), None if d2t is None else i32(d2t, dev), V,
                           i32(pos, dev), pos_out, acc, ne, emit, nt, st)
    torch.cuda.synchronize()
    return dict(pos_out=pos_out.cpu().numpy(), accept_len=acc.cpu().numpy(), n_emit=ne.cpu().numpy(),
                emit=emit.cpu().numpy(), next_tok=nt.cpu().numpy(), status=st.cpu().numpy())


def assert_accept_equal(got, ref, what):
    for key in ("status", "accept_len", "n_emit", "pos_out", "next_tok", "emit"):
        assert np.array_equal(got[key], ref[key]), f"{what}: {key} gpu {got[key]} ref {ref[key]}"


# ---------------------------------------------------------------------------
# tree rows
# ---------------------------------------------------------------------------
def gpu_attn_tree(x: synth.VerifyInputs, parent, dev, kv_split_tokens=0, k=None, k_pool=None, v_pool=None):
    """Runs spec_verify_attn_tree; returns (out bf16 device, k_pool, v_pool, status np)."""
    import greedy_draft_verify_amd as gdv
    k = x.k if k is None else k
    R = x.q.shape[0]
    kp = (x.k_pool if k_pool is None else k_pool).to(dev).clone()
    vp = (x.v_pool if v_pool is None else v_pool).to(dev).clone()
    out = torch.full((R, x.wl.Hq, x.wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    status = torch.full((len(x.pos),), -7, dtype=torch.int32, device=dev)
    gdv.spec_verify_attn_tree(x.q.to(dev).contiguous(), x.k_new.to(dev).contiguous(), x.v_new.to(dev).contiguous(),
                              kp, vp, i32(x.page_table, dev), i32(x.pos, dev), i32(k, dev), i32(parent, dev), x.scale,
                              out, status, kv_split_tokens=kv_split_tokens)
    torch.cuda.synchronize()
    return out, kp, vp, status.cpu().numpy()


def oracle_attn_tree(x: synth.VerifyInputs, parent, seqs=None):
    """Oracle tree attention for the selected sequences: (rows, out fp64, k_pool, v_pool, status)."""
    wl = x.wl
    B = len(x.pos)
    seqs = list(range(B)) if seqs is None else list(seqs)
    off_all = np.concatenate([[0], np.cumsum(x.k + 1)]).astype(np.int64)
    rows = np.concatenate([np.arange(off_all[s], off_all[s + 1]) for s in seqs])
    kp, vp = bits(x.k_pool).copy(), bits(x.v_pool).copy()
    pos, k, pt = x.pos[seqs], x.k[seqs], x.page_table[seqs]
    par = np.ascontiguousarray(np.asarray(parent)[seqs], np.int32)
    kmax = par.shape[1] - 1
    qb, knb, vnb = bits(x.q)[rows], bits(x.k_new)[rows], bits(x.v_new)[rows]
    R = len(rows)
    off, st = oracle.validate(pt, pt.shape[1], x.n_pages, pos, k, kmax, len(seqs), R)
    oracle.validate_tree(par, kmax, k, len(seqs), st)
    oracle.append_kv(knb, vnb, kp, vp, pt, pt.shape[1], pos, k, off, st, len(seqs), wl.Hkv, wl.D)
    out = oracle.verify_attn_tree(qb, kp, vp, pt, pt.shape[1], pos, k, par, kmax, off, st, len(seqs), R, wl.Hq,
                                  wl.Hkv, wl.D, x.scale)
    return rows, out, kp, vp, st


def gpu_tree_accept(g, drafts, k, parent, d2t, V, pos, dev):
    import greedy_draft_verify_amd as gdv
    B = len(k)
    drafts = np.ascontiguousarray(drafts, np.int32)
    kmax = drafts.shape[1]
    z = lambda: torch.full((B,), -9, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = z(), z(), z(), z(), z()
    emit = torch.full((B, kmax + 1), -9, dtype=torch.int32, device=dev)
    path = torch.full((B, kmax), -9, dtype=torch.int32, device=dev)
    gdv.spec_tree_accept(i32(g, dev), i32(drafts, dev), i32(k, dev), i32(parent, dev),
                         None if d2t is None else i32(d2t, dev), V, i32(pos, dev), pos_out, acc, ne, emit, nt, path, st)
    torch.cuda.synchronize()
    return dict(pos_out=pos_out.cpu().numpy(), accept_len=acc.cpu().numpy(), n_emit=ne.cpu().numpy(),
                emit=emit.cpu().numpy(), next_tok=nt.cpu().numpy(), path=path.cpu().numpy(),
                status=st.cpu().numpy())
