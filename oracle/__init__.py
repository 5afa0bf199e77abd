"""ctypes front end of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library and
its Python binding) never does. Arrays are numpy: bf16 tensors travel as their
raw ``uint16`` bit patterns, everything the oracle computes comes back in fp64.

Functions mirror the definitions in ``oracle.c``; see the comments there for the
passages of the pages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

# Status bits, as the public header documents them for the library.
BAD_PAGE, BAD_POS, BAD_ROWS, BAD_TOKEN, BAD_TREE, BAD_LIMIT = 1, 2, 4, 8, 16, 32
PAGE = 16


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                        "-ffp-contract=off", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def validate(page_table, max_pages, n_pages, pos, k, kmax, B, R):
    off = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    pt = None if page_table is None else _i32(page_table)
    lib().oracle_validate(_p(pt), ctypes.c_int32(max_pages), ctypes.c_int64(n_pages), _p(_i32(pos)),
                          _p(_i32(k)), ctypes.c_int32(kmax), ctypes.c_int32(B), ctypes.c_int32(R),
                          _p(off), _p(st))
    return off, st


def append_kv(k_new, v_new, k_pool, v_pool, page_table, max_pages, pos, k, off, st, B, Hkv, D):
    """In place on k_pool / v_pool (uint16 arrays)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    lib().oracle_append_kv(_p(_u16(k_new)), _p(_u16(v_new)), _p(k_pool), _p(v_pool),
                           _p(_i32(page_table)), ctypes.c_int32(max_pages), _p(_i32(pos)),
                           _p(_i32(k)), _p(_i32(off)), _p(_i32(st)), ctypes.c_int32(B),
                           ctypes.c_int32(Hkv), ctypes.c_int32(D))


def verify_attn(q, k_pool, v_pool, page_table, max_pages, pos, k, off, st, B, R, Hq, Hkv, D, scale,
                out=None):
    """Returns fp64 [R, Hq, D]; rows of bad sequences keep ``out``'s values (NaN if new)."""
    if out is None:
        out = np.full((R, Hq, D), np.nan, np.float64)
    lib().oracle_verify_attn(_p(_u16(q)), _p(_u16(k_pool)), _p(_u16(v_pool)), _p(_i32(page_table)),
                             ctypes.c_int32(max_pages), _p(_i32(pos)), _p(_i32(k)), _p(_i32(off)),
                             _p(_i32(st)), ctypes.c_int32(B), ctypes.c_int32(R), ctypes.c_int32(Hq),
                             ctypes.c_int32(Hkv), ctypes.c_int32(D), ctypes.c_double(scale), _p(out))
    return out


def lm_head_logits(hidden, w, R, H, V, chunk=16384):
    """logit[r, v] = sum_i w[v, i] hidden[r, i] in fp64 (numpy's matmul as the contraction
    step, one vocabulary chunk at a time; inputs widened exactly from bf16)."""
    h = bf16_bits_to_f64(np.asarray(hidden).reshape(R, H))
    wv = np.asarray(w).reshape(V, H)
    out = np.empty((R, V), np.float64)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = h @ bf16_bits_to_f64(wv[v0:v0 + chunk]).T
    return out


def argmax_rows(logits):
    """First maximum, its value and the runner-up value per row (plain C scan)."""
    logits = np.ascontiguousarray(logits, np.float64)
    R, V = logits.shape
    g = np.zeros(R, np.int32)
    t1 = np.zeros(R, np.float64)
    t2 = np.zeros(R, np.float64)
    lib().oracle_argmax_rows(_p(logits), ctypes.c_int32(R), ctypes.c_int32(V), _p(g), _p(t1), _p(t2))
    return g, t1, t2


def lm_head_argmax(hidden, w, R, H, V, want_logits=False):
    """Returns (g int32 [R], top1 f64 [R], top2 f64 [R], logits f64 [R,V] or None)."""
    lg = lm_head_logits(hidden, w, R, H, V)
    g, t1, t2 = argmax_rows(lg)
    return g, t1, t2, (lg if want_logits else None)


def lm_head_argmax_loops(hidden, w, R, H, V, want_logits=False):
    """The same definition as plain C loops (an independent implementation, for pins)."""
    g = np.zeros(R, np.int32)
    t1 = np.zeros(R, np.float64)
    t2 = np.zeros(R, np.float64)
    lg = np.zeros((R, V), np.float64) if want_logits else None
    lib().oracle_lm_head_argmax(_p(_u16(hidden)), _p(_u16(w)), ctypes.c_int32(R), ctypes.c_int32(H),
                                ctypes.c_int32(V), _p(g), _p(t1), _p(t2), _p(lg))
    return g, t1, t2, lg


def greedy_accept(g, drafts, kmax, k, d2t, n_draft_vocab, V, B, R, pos_in):
    """Returns dict with pos_out, accept_len, n_emit, emit [B, kmax+1], next_tok, status."""
    pos_out = np.zeros(B, np.int32)
    acc = np.zeros(B, np.int32)
    ne = np.zeros(B, np.int32)
    emit = np.zeros((B, kmax + 1), np.int32)
    nt = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    dr = _i32(drafts).reshape(B, max(kmax, 0)) if kmax > 0 else np.zeros((B, 1), np.int32)
    d2 = None if d2t is None else _i32(d2t)
    lib().oracle_greedy_accept(_p(_i32(g)), _p(dr), ctypes.c_int32(kmax), _p(_i32(k)), _p(d2),
                               ctypes.c_int32(n_draft_vocab), ctypes.c_int32(V), ctypes.c_int32(B),
                               ctypes.c_int32(R), _p(_i32(pos_in)), _p(pos_out), _p(acc), _p(ne),
                               _p(emit), _p(nt), _p(st))
    return dict(pos_out=pos_out, accept_len=acc, n_emit=ne, emit=emit, next_tok=nt, status=st)


def delta_verify(q, k, v, a, b, q_scale, state, B, T, Hd, dk, dv):
    """Returns (rec f64 [B,T,Hd,dv,dk], o f64 [B,T,Hd,dv])."""
    rec = np.zeros((B, T, Hd, dv, dk), np.float64)
    o = np.zeros((B, T, Hd, dv), np.float64)
    lib().oracle_delta_verify(_p(_u16(q)), _p(_u16(k)), _p(_u16(v)),
                              _p(np.ascontiguousarray(a, np.float32)),
                              _p(np.ascontiguousarray(b, np.float32)), ctypes.c_double(q_scale),
                              _p(np.ascontiguousarray(state, np.float32)), ctypes.c_int32(B),
                              ctypes.c_int32(T), ctypes.c_int32(Hd), ctypes.c_int32(dk),
                              ctypes.c_int32(dv), _p(rec), _p(o))
    return rec, o


def delta_rollback(rec, L, state, B, T, Hd, dk, dv):
    """state: fp64 [B,Hd,dv,dk], updated in place and returned."""
    state = np.ascontiguousarray(state, np.float64)
    lib().oracle_delta_rollback(_p(np.ascontiguousarray(rec, np.float64)), _p(_i32(L)),
                                ctypes.c_int32(B), ctypes.c_int32(T), ctypes.c_int32(Hd),
                                ctypes.c_int32(dk), ctypes.c_int32(dv), _p(state))
    return state


# ---------------------------------------------------------------------------
# tree verify (fast.py _set_rows / _tree_cycle): rows = nodes in creation order,
# parent [B][kmax + 1] with parent[s][0] = -1 and parent[s][i] in [0, i)
def validate_tree(parent, kmax, k, B, st):
    """ORs BAD_TREE into st (int32 [B], in place) where the parent list is not a tree."""
    assert st.dtype == np.int32 and st.flags.c_contiguous
    lib().oracle_validate_tree(_p(_i32(parent).reshape(B, kmax + 1)), ctypes.c_int32(kmax), _p(_i32(k)),
                               ctypes.c_int32(B), _p(st))
    return st


def verify_attn_tree(q, k_pool, v_pool, page_table, max_pages, pos, k, parent, kmax, off, st, B, R, Hq, Hkv,
                     D, scale, out=None):
    """Tree rows: returns fp64 [R, Hq, D] (rows of bad sequences keep ``out``'s values)."""
    if out is None:
        out = np.full((R, Hq, D), np.nan, np.float64)
    lib().oracle_verify_attn_tree(_p(_u16(q)), _p(_u16(k_pool)), _p(_u16(v_pool)), _p(_i32(page_table)),
                                  ctypes.c_int32(max_pages), _p(_i32(pos)), _p(_i32(k)),
                                  _p(_i32(parent).reshape(B, kmax + 1)), ctypes.c_int32(kmax),
                                  _p(_i32(off)), _p(_i32(st)), ctypes.c_int32(B), ctypes.c_int32(Hq),
                                  ctypes.c_int32(Hkv), ctypes.c_int32(D), ctypes.c_double(scale), _p(out))
    return out


def tree_accept(g, drafts, kmax, k, parent, d2t, n_draft_vocab, V, B, R, pos_in):
    """Returns dict with pos_out, accept_len, n_emit, emit [B, kmax+1], next_tok, path [B, kmax], status."""
    pos_out = np.zeros(B, np.int32)
    acc = np.zeros(B, np.int32)
    ne = np.zeros(B, np.int32)
    emit = np.zeros((B, kmax + 1), np.int32)
    nt = np.zeros(B, np.int32)
    path = np.zeros((B, max(kmax, 1)), np.int32)
    st = np.zeros(B, np.int32)
    dr = _i32(drafts).reshape(B, max(kmax, 0)) if kmax > 0 else np.zeros((B, 1), np.int32)
    d2 = None if d2t is None else _i32(d2t)
    lib().oracle_tree_accept(_p(_i32(g)), _p(dr), ctypes.c_int32(kmax), _p(_i32(k)),
                             _p(_i32(parent).reshape(B, kmax + 1)), _p(d2), ctypes.c_int32(n_draft_vocab),
                             ctypes.c_int32(V), ctypes.c_int32(B), ctypes.c_int32(R), _p(_i32(pos_in)),
                             _p(pos_out), _p(acc), _p(ne), _p(emit), _p(nt), _p(path), _p(st))
    return dict(pos_out=pos_out, accept_len=acc, n_emit=ne, emit=emit, next_tok=nt, path=path[:, :kmax],
                status=st)


def kv_compact(k_pool, v_pool, page_table, max_pages, pos, path, accept_len, kmax, st, B, Hkv, D):
    """In place on k_pool / v_pool (uint16 arrays)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    ph = _i32(path).reshape(B, kmax) if kmax > 0 else np.zeros((B, 1), np.int32)
    lib().oracle_kv_compact(_p(k_pool), _p(v_pool), _p(_i32(page_table)), ctypes.c_int32(max_pages),
                            _p(_i32(pos)), _p(ph), _p(_i32(accept_len)), ctypes.c_int32(kmax), _p(_i32(st)),
                            ctypes.c_int32(B), ctypes.c_int32(Hkv), ctypes.c_int32(D))


# ---------------------------------------------------------------------------
# speculative-sampling verify (DSSD fast.py _sample_verify)
def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: ctr 4 uint32 words, key 2 uint32 words -> 4 uint32 words."""
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def accept_uniform(row_ctr, seed):
    f = lib().oracle_accept_uniform
    f.restype = ctypes.c_double
    return f(_p(np.ascontiguousarray(row_ctr, np.int32)), ctypes.c_uint64(seed))


def sample_rows(logits, T, q_tok, q_prob, row_ctr, seed):
    """logits fp64 [R, V]; q_tok int32 [R, NQ]; q_prob fp32 [R, NQ]; row_ctr int32 [R, 2].
    Returns dict lse [R], z_supp [R, NQ], sample_p [R], sample_res [R], and gap_p / gap_res
    [R]: how far each draw's winner is above the runner-up (in log-weight + noise)."""
    logits = np.ascontiguousarray(logits, np.float64)
    R, V = logits.shape
    q_tok = _i32(q_tok)
    NQ = q_tok.shape[1]
    q_prob = np.ascontiguousarray(q_prob, np.float32)
    lse = np.zeros(R, np.float64)
    z = np.zeros((R, NQ), np.float64)
    sp = np.zeros(R, np.int32)
    sr = np.zeros(R, np.int32)
    gp = np.zeros(R, np.float64)
    gr = np.zeros(R, np.float64)
    lib().oracle_sample_rows(_p(logits), ctypes.c_int32(R), ctypes.c_int32(V), ctypes.c_double(T), _p(q_tok),
                             _p(q_prob), ctypes.c_int32(NQ), _p(_i32(row_ctr)), ctypes.c_uint64(seed), _p(lse),
                             _p(z), _p(sp), _p(sr), _p(gp), _p(gr))
    return dict(lse=lse, z_supp=z, sample_p=sp, sample_res=sr, gap_p=gp, gap_res=gr)


def sample_accept(drafts, kmax, k, d2t, n_draft_vocab, V, B, R, q_tok, q_prob, rows, row_ctr, seed, pos_in):
    """rows: the dict of sample_rows. Returns the same dict as greedy_accept."""
    q_tok = _i32(q_tok)
    NQ = q_tok.shape[1]
    pos_out = np.zeros(B, np.int32)
    acc = np.zeros(B, np.int32)
    ne = np.zeros(B, np.int32)
    emit = np.zeros((B, kmax + 1), np.int32)
    nt = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    dr = _i32(drafts).reshape(B, max(kmax, 0)) if kmax > 0 else np.zeros((B, 1), np.int32)
    d2 = None if d2t is None else _i32(d2t)
    lib().oracle_sample_accept(_p(dr), ctypes.c_int32(kmax), _p(_i32(k)), _p(d2), ctypes.c_int32(n_draft_vocab),
                               ctypes.c_int32(V), ctypes.c_int32(B), ctypes.c_int32(R), _p(q_tok),
                               _p(np.ascontiguousarray(q_prob, np.float32)), ctypes.c_int32(NQ),
                               _p(np.ascontiguousarray(rows["lse"], np.float64)),
                               _p(np.ascontiguousarray(rows["z_supp"], np.float64)), _p(_i32(rows["sample_p"])),
                               _p(_i32(rows["sample_res"])), _p(_i32(row_ctr)), ctypes.c_uint64(seed),
                               _p(_i32(pos_in)), _p(pos_out), _p(acc), _p(ne), _p(emit), _p(nt), _p(st))
    return dict(pos_out=pos_out, accept_len=acc, n_emit=ne, emit=emit, next_tok=nt, status=st)


def sample_accept_dense(drafts, kmax, k, d2t, n_draft_vocab, V, B, R, logits, T, q, row_ctr, seed, pos_in,
                        rel=0.0):
    """Speculative sampling with a dense draft distribution q [R, V] (fp32) over the target
    vocabulary; logits fp64 [R, V]. Returns the greedy_accept dict plus margin [B] (how
    decided the acceptance tests are, in log(u) vs log(p/q)) and gap [B] (how decided the
    deciding draw is when p is known to relative precision rel; <= 0: not decided)."""
    logits = np.ascontiguousarray(logits, np.float64)
    q = np.ascontiguousarray(q, np.float32)
    assert logits.shape == (R, V) and q.shape == (R, V)
    pos_out, acc, ne, nt, st = (np.zeros(B, np.int32) for _ in range(5))
    emit = np.zeros((B, kmax + 1), np.int32)
    margin = np.zeros(B, np.float64)
    gap = np.zeros(B, np.float64)
    dr = _i32(drafts).reshape(B, max(kmax, 0)) if kmax > 0 else np.zeros((B, 1), np.int32)
    d2 = None if d2t is None else _i32(d2t)
    lib().oracle_sample_accept_dense(_p(dr), ctypes.c_int32(kmax), _p(_i32(k)), _p(d2),
                                     ctypes.c_int32(n_draft_vocab), ctypes.c_int32(V), ctypes.c_int32(B),
                                     ctypes.c_int32(R), _p(logits), ctypes.c_double(T), _p(q), _p(_i32(row_ctr)),
                                     ctypes.c_uint64(seed), _p(_i32(pos_in)), _p(pos_out), _p(acc), _p(ne), _p(emit),
                                     _p(nt), _p(st), ctypes.c_double(rel), _p(margin), _p(gap))
    return dict(pos_out=pos_out, accept_len=acc, n_emit=ne, emit=emit, next_tok=nt, status=st, margin=margin,
                gap=gap)


def greedy_accept_stop(g, drafts, kmax, k, d2t, n_draft_vocab, V, B, R, stop_ids, remaining, pos_in):
    """Greedy acceptance truncated at the first stop token and at remaining[s] tokens
    (remaining None: no limit). Returns the greedy_accept dict plus done [B]."""
    pos_out = np.zeros(B, np.int32)
    acc = np.zeros(B, np.int32)
    ne = np.zeros(B, np.int32)
    emit = np.zeros((B, kmax + 1), np.int32)
    nt = np.zeros(B, np.int32)
    done = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    dr = _i32(drafts).reshape(B, max(kmax, 0)) if kmax > 0 else np.zeros((B, 1), np.int32)
    d2 = None if d2t is None else _i32(d2t)
    stops = _i32(stop_ids) if len(stop_ids) else np.zeros(1, np.int32)
    rem = None if remaining is None else _i32(remaining)
    lib().oracle_greedy_accept_stop(_p(_i32(g)), _p(dr), ctypes.c_int32(kmax), _p(_i32(k)), _p(d2),
                                    ctypes.c_int32(n_draft_vocab), ctypes.c_int32(V), ctypes.c_int32(B),
                                    ctypes.c_int32(R), _p(stops), ctypes.c_int32(len(stop_ids)), _p(rem),
                                    _p(_i32(pos_in)), _p(pos_out), _p(acc), _p(ne), _p(emit), _p(nt), _p(done),
                                    _p(st))
    return dict(pos_out=pos_out, accept_len=acc, n_emit=ne, emit=emit, next_tok=nt, done=done, status=st)


def truncate_stop(res, kmax, stop_ids, remaining, pos_in, path=None):
    """Stop tokens and a limit applied to an acceptance walk's outputs (a dict as the
    accept functions return; copied). path: the tree walk's path [B, kmax] or None."""
    out = {k: np.ascontiguousarray(v, np.int32).copy() for k, v in res.items()}
    B = len(out["n_emit"])
    done = np.zeros(B, np.int32)
    stops = _i32(stop_ids) if len(stop_ids) else np.zeros(1, np.int32)
    rem = None if remaining is None else _i32(remaining)
    ph = None if path is None else np.ascontiguousarray(path, np.int32).reshape(B, kmax).copy()
    lib().oracle_truncate_stop(_p(out["emit"]), _p(out["n_emit"]), _p(out["accept_len"]), _p(_i32(pos_in)),
                               _p(out["pos_out"]), _p(out["next_tok"]), _p(ph), ctypes.c_int32(kmax), _p(stops),
                               ctypes.c_int32(len(stop_ids)), _p(rem), _p(done), _p(out["status"]), ctypes.c_int32(B))
    out["done"] = done
    if ph is not None:
        out["path"] = ph
    return out
