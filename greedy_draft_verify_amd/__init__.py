"""Python binding of libspecverify.so, the MI355X verify-step library.

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch
supplies device memory (tensors are passed as raw pointers) and the stream (the
current torch stream unless one is given). The functions keep the C names and
argument order of ``include/spec_verify.h``; shapes are read off the tensors.

The library must have been built (``python -m greedy_draft_verify_amd.build`` or
``__graft_entry__.build()``); there is no fallback path, a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_PAGE_TOKENS = 16
STATUS_BAD_PAGE, STATUS_BAD_POS, STATUS_BAD_ROWS, STATUS_BAD_TOKEN = 1, 2, 4, 8
DELTA_RECORD, DELTA_ROLLBACK, DELTA_BOTH, DELTA_VERIFY, DELTA_RESCAN = 1, 2, 3, 4, 5

EXPORTED = ["spec_version", "spec_last_error", "spec_attn_split_tokens",
            "spec_verify_attn_workspace_bytes", "spec_verify_attn",
            "spec_lm_head_argmax_workspace_bytes", "spec_lm_head_argmax", "spec_lm_head_argmax_noalloc",
            "spec_lm_head_argmax_accept",
            "spec_lm_head_packed_bytes",
            "spec_lm_head_pack", "spec_greedy_accept", "spec_delta_verify_rollback",
            "spec_verify_attn_tree_workspace_bytes", "spec_verify_attn_tree", "spec_tree_accept",
            "spec_kv_compact", "spec_lm_head_sample_workspace_bytes", "spec_lm_head_sample",
            "spec_sample_accept", "spec_lm_head_sample_dense", "spec_sample_accept_dense_workspace_bytes",
            "spec_sample_accept_dense", "spec_greedy_accept_stop", "spec_truncate_stop", "spec_kpolicy_init", "spec_kpolicy_accept_prob",
            "spec_kpolicy_verify_cost", "spec_kpolicy_expected_tokens", "spec_kpolicy_choose",
            "spec_kpolicy_update", "spec_kpolicy_update_batch"]

SPEC_KPOLICY_MAXK, SPEC_KPOLICY_MAXPTS = 64, 32


class _KPolicyStruct(ctypes.Structure):
    """Mirror of the header's spec_kpolicy."""
    _fields_ = [("kmin", ctypes.c_int32), ("kmax", ctypes.c_int32), ("prior_p", ctypes.c_double),
                ("prior_n", ctypes.c_double), ("draft_us", ctypes.c_double), ("n_points", ctypes.c_int32),
                ("cost_rows", ctypes.c_double * SPEC_KPOLICY_MAXPTS), ("cost_us", ctypes.c_double * SPEC_KPOLICY_MAXPTS),
                ("tried", ctypes.c_double * SPEC_KPOLICY_MAXK), ("kept", ctypes.c_double * SPEC_KPOLICY_MAXK)]

_lib = None


class SpecError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Loads the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SpecError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        L.spec_version.restype = ctypes.c_int
        L.spec_last_error.restype = ctypes.c_char_p
        L.spec_attn_split_tokens.argtypes = [i32]
        L.spec_attn_split_tokens.restype = i32
        L.spec_verify_attn_workspace_bytes.argtypes = [i32] * 7
        L.spec_verify_attn_workspace_bytes.restype = sz
        L.spec_verify_attn.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                       f32, i32, vp, vp, sz, vp, vp]
        L.spec_lm_head_argmax_workspace_bytes.argtypes = [i32, i32, i32]
        L.spec_lm_head_argmax_workspace_bytes.restype = sz
        L.spec_lm_head_argmax.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.spec_lm_head_argmax_noalloc.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
        L.spec_lm_head_argmax_accept.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp, i32, i32, vp, vp,
                                                 vp, vp, vp, vp, vp, vp, sz, vp]
        L.spec_lm_head_packed_bytes.argtypes = [i32, i32]
        L.spec_lm_head_packed_bytes.restype = sz
        L.spec_lm_head_pack.argtypes = [vp, i32, i32, vp, vp]
        L.spec_greedy_accept.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                         vp, vp]
        L.spec_delta_verify_rollback.argtypes = [i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, i32, i32, i32, i32,
                                                 i32, vp, vp]
        L.spec_verify_attn_tree_workspace_bytes.argtypes = [i32] * 8
        L.spec_verify_attn_tree_workspace_bytes.restype = sz
        L.spec_verify_attn_tree.argtypes = [vp, vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                            i32, f32, i32, vp, vp, sz, vp, vp]
        L.spec_tree_accept.argtypes = [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp]
        L.spec_kv_compact.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, i32, i32, i32, i32, vp, vp]
        u64 = ctypes.c_uint64
        L.spec_lm_head_sample_workspace_bytes.argtypes = [i32, i32, i32]
        L.spec_lm_head_sample_workspace_bytes.restype = sz
        L.spec_lm_head_sample.argtypes = [vp, vp, i32, i32, i32, f32, vp, vp, i32, vp, u64, vp, vp, vp, vp, vp, sz,
                                          vp]
        L.spec_sample_accept.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, u64,
                                         vp, vp, vp, vp, vp, vp, vp, vp]
        L.spec_greedy_accept_stop.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp]
        L.spec_lm_head_sample_dense.argtypes = [vp, vp, i32, i32, i32, f32, vp, u64, vp, vp, vp, vp, sz, vp]
        L.spec_sample_accept_dense_workspace_bytes.argtypes = [i32]
        L.spec_sample_accept_dense_workspace_bytes.restype = sz
        L.spec_sample_accept_dense.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, u64, vp, vp,
                                               vp, vp, vp, vp, vp, vp, sz, vp]
        L.spec_truncate_stop.argtypes = [i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        pp = ctypes.POINTER(_KPolicyStruct)
        dbl, dp = ctypes.c_double, ctypes.POINTER(ctypes.c_double)
        L.spec_kpolicy_init.argtypes = [pp, i32, i32, dbl, dbl, dbl, dp, dp, i32]
        L.spec_kpolicy_init.restype = ctypes.c_int
        for name, args in (("spec_kpolicy_accept_prob", [pp, i32]), ("spec_kpolicy_verify_cost", [pp, dbl]),
                           ("spec_kpolicy_expected_tokens", [pp, i32])):
            getattr(L, name).argtypes = args
            getattr(L, name).restype = dbl
        L.spec_kpolicy_choose.argtypes = [pp, i32, i32]
        L.spec_kpolicy_choose.restype = i32
        L.spec_kpolicy_update.argtypes = [pp, i32, i32]
        L.spec_kpolicy_update.restype = None
        L.spec_kpolicy_update_batch.argtypes = [pp, vp, vp, i32]
        L.spec_kpolicy_update_batch.restype = ctypes.c_int
        for name in ("spec_greedy_accept_stop", "spec_truncate_stop", "spec_lm_head_sample_dense",
                     "spec_sample_accept_dense", "spec_verify_attn", "spec_lm_head_argmax", "spec_lm_head_pack",
                     "spec_greedy_accept",
                     "spec_delta_verify_rollback", "spec_verify_attn_tree", "spec_tree_accept",
                     "spec_kv_compact", "spec_lm_head_sample", "spec_sample_accept"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> int:
    return lib().spec_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int, name: str):
    if rc != 0:
        msg = lib().spec_last_error().decode(errors="replace")
        raise SpecError(f"{name} returned {rc}: {msg}")


def _want(t, dtype, name, ndim=None):
    if t is None:
        raise SpecError(f"{name} is required")
    if t.dtype != dtype:
        raise SpecError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise SpecError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise SpecError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise SpecError(f"{name}: {t.dim()} dims, expected {ndim}")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise SpecError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def attn_split_tokens(max_pages: int) -> int:
    return lib().spec_attn_split_tokens(max_pages)


def verify_attn_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kv_split_tokens=0) -> int:
    return lib().spec_verify_attn_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kv_split_tokens)


def verify_attn_tree_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kmax, kv_split_tokens=0) -> int:
    return lib().spec_verify_attn_tree_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kv_split_tokens, kmax)


def lm_head_argmax_workspace_bytes(R, H, V) -> int:
    return lib().spec_lm_head_argmax_workspace_bytes(R, H, V)


def workspace(nbytes: int, device="cuda", zero: bool = False) -> torch.Tensor:
    """A workspace buffer; spec_lm_head_argmax needs one that is zero on first use."""
    n = max(int(nbytes), 1)
    if zero:
        return torch.zeros(n, dtype=torch.uint8, device=device)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _attn_shapes(q, k_new, v_new, k_pool, v_pool, page_table, pos, k, out, seq_status):
    for t, n, nd in ((q, "q", 3), (k_new, "k_new", 3), (v_new, "v_new", 3), (k_pool, "k_pool", 3),
                     (v_pool, "v_pool", 3), (out, "out", 3)):
        _want(t, torch.bfloat16, n, nd)
    for t, n in ((page_table, "page_table"), (pos, "pos"), (k, "k"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    R, Hq, D = q.shape
    Hkv = k_new.shape[1]
    _want(page_table, torch.int32, "page_table", 2)
    B, max_pages = page_table.shape
    n_pages = k_pool.shape[0]
    _shape(k_new, (R, Hkv, D), "k_new")
    _shape(v_new, (R, Hkv, D), "v_new")
    _shape(k_pool, (n_pages, Hkv, SPEC_PAGE_TOKENS * D), "k_pool")
    _shape(v_pool, (n_pages, Hkv, SPEC_PAGE_TOKENS * D), "v_pool")
    _shape(out, (R, Hq, D), "out")
    for t, n in ((pos, "pos"), (k, "k"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    return R, Hq, Hkv, D, B, max_pages, n_pages


def spec_verify_attn(q, k_new, v_new, k_pool, v_pool, page_table, pos, k, kmax, scale, out, seq_status,
                     workspace_buf=None, kv_split_tokens=0, stream=None):
    """q [R,Hq,D], k_new/v_new [R,Hkv,D], k_pool/v_pool [n_pages,Hkv,16*D] (pool block layout),
    out [R,Hq,D] (bf16); page_table [B,max_pages], pos [B], k [B], seq_status [B] (int32);
    kmax = an upper bound on k."""
    R, Hq, Hkv, D, B, max_pages, n_pages = _attn_shapes(q, k_new, v_new, k_pool, v_pool, page_table, pos, k,
                                                        out, seq_status)
    if workspace_buf is None:
        workspace_buf = workspace(verify_attn_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kv_split_tokens),
                                  q.device)
    rc = lib().spec_verify_attn(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), n_pages,
                                _ptr(page_table), max_pages, _ptr(pos), _ptr(k), kmax, B, R, Hq, Hkv, D, scale,
                                kv_split_tokens, _ptr(out), _ptr(workspace_buf), workspace_buf.numel(),
                                _ptr(seq_status), _stream(stream))
    _check(rc, "spec_verify_attn")


def spec_verify_attn_tree(q, k_new, v_new, k_pool, v_pool, page_table, pos, k, parent, scale, out, seq_status,
                          workspace_buf=None, kv_split_tokens=0, stream=None):
    """Tree rows: as spec_verify_attn, plus parent [B, kmax+1] int32 (parent[s][0] = -1,
    parent[s][i] in [0, i)); kmax = parent.shape[1] - 1."""
    R, Hq, Hkv, D, B, max_pages, n_pages = _attn_shapes(q, k_new, v_new, k_pool, v_pool, page_table, pos, k,
                                                        out, seq_status)
    _want(parent, torch.int32, "parent", 2)
    if parent.shape[0] != B:
        raise SpecError(f"parent: {tuple(parent.shape)}, expected ({B}, kmax + 1)")
    kmax = parent.shape[1] - 1
    if workspace_buf is None:
        workspace_buf = workspace(verify_attn_tree_workspace_bytes(B, R, Hq, Hkv, D, max_pages, kmax,
                                                                   kv_split_tokens), q.device)
    rc = lib().spec_verify_attn_tree(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), n_pages,
                                     _ptr(page_table), max_pages, _ptr(pos), _ptr(k), _ptr(parent), kmax, B, R,
                                     Hq, Hkv, D, scale, kv_split_tokens, _ptr(out), _ptr(workspace_buf),
                                     workspace_buf.numel(), _ptr(seq_status), _stream(stream))
    _check(rc, "spec_verify_attn_tree")


def spec_tree_accept(argmax, drafts, k, parent, d2t, V, pos_in, pos_out, accept_len, n_emit, emit, next_tok,
                     path, seq_status, stream=None):
    """Tree acceptance walk: as spec_greedy_accept, plus parent [B, kmax+1] and the output
    path [B, kmax] (int32)."""
    for t, n in ((argmax, "argmax"), (drafts, "drafts"), (k, "k"), (parent, "parent"), (pos_in, "pos_in"),
                 (pos_out, "pos_out"), (accept_len, "accept_len"), (n_emit, "n_emit"), (emit, "emit"),
                 (next_tok, "next_tok"), (path, "path"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    _want(drafts, torch.int32, "drafts", 2)
    B, kmax = drafts.shape
    R = argmax.shape[0]
    _shape(argmax, (R,), "argmax")
    _shape(parent, (B, kmax + 1), "parent")
    _shape(emit, (B, kmax + 1), "emit")
    _shape(path, (B, kmax), "path")
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    rc = lib().spec_tree_accept(_ptr(argmax), _ptr(drafts), kmax, _ptr(k), _ptr(parent), _ptr(d2t),
                                0 if d2t is None else d2t.shape[0], V, B, R, _ptr(pos_in), _ptr(pos_out),
                                _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok), _ptr(path),
                                _ptr(seq_status), _stream(stream))
    _check(rc, "spec_tree_accept")


def spec_kv_compact(k_pool, v_pool, page_table, pos, path, accept_len, seq_status, stream=None):
    """Moves slot pos + path[s][d] to pos + 1 + d (every kv head) for the sequences whose
    seq_status is 0 (in/out); k_pool/v_pool [n_pages,Hkv,16*D] bf16, path [B,kmax] int32."""
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _want(t, torch.bfloat16, n, 3)
    for t, n in ((page_table, "page_table"), (pos, "pos"), (path, "path"), (accept_len, "accept_len"),
                 (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    _want(page_table, torch.int32, "page_table", 2)
    _want(path, torch.int32, "path", 2)
    B, max_pages = page_table.shape
    n_pages, Hkv, blk = k_pool.shape
    D = blk // SPEC_PAGE_TOKENS
    _shape(v_pool, (n_pages, Hkv, blk), "v_pool")
    kmax = path.shape[1]
    _shape(path, (B, kmax), "path")
    for t, n in ((pos, "pos"), (accept_len, "accept_len"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    rc = lib().spec_kv_compact(_ptr(k_pool), _ptr(v_pool), n_pages, _ptr(page_table), max_pages, _ptr(pos),
                               _ptr(path), _ptr(accept_len), kmax, B, Hkv, D, _ptr(seq_status), _stream(stream))
    _check(rc, "spec_kv_compact")


def lm_head_packed_bytes(V, H) -> int:
    return lib().spec_lm_head_packed_bytes(V, H)


def spec_lm_head_pack(w, w_packed=None, stream=None):
    """w [V,H] bf16 (row-major) -> packed weight (a flat bf16 tensor) for spec_lm_head_argmax."""
    _want(w, torch.bfloat16, "w", 2)
    V, H = w.shape
    nbytes = lm_head_packed_bytes(V, H)
    if w_packed is None:
        w_packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    if w_packed.numel() * 2 != nbytes:
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {nbytes}")
    rc = lib().spec_lm_head_pack(_ptr(w), V, H, _ptr(w_packed), _stream(stream))
    _check(rc, "spec_lm_head_pack")
    return w_packed


def spec_lm_head_argmax(hidden, w_packed, V, argmax, maxval=None, workspace_buf=None, stream=None):
    """hidden [R,H] bf16, w_packed from spec_lm_head_pack (vocabulary V) -> argmax [R] int32,
    maxval [R] fp32 (optional). A workspace_buf must be zero on its first use (every call
    leaves it zero) and must not be shared by calls that may overlap."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    _want(argmax, torch.int32, "argmax", 1)
    if maxval is not None:
        _want(maxval, torch.float32, "maxval", 1)
    R, H = hidden.shape
    if w_packed.numel() * 2 != lm_head_packed_bytes(V, H):
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {lm_head_packed_bytes(V, H)} "
                        f"for V={V} H={H}")
    _shape(argmax, (R,), "argmax")
    if maxval is not None:
        _shape(maxval, (R,), "maxval")
    if workspace_buf is None:
        workspace_buf = workspace(lm_head_argmax_workspace_bytes(R, H, V), hidden.device, zero=True)
    rc = lib().spec_lm_head_argmax(_ptr(hidden), _ptr(w_packed), R, H, V, _ptr(argmax), _ptr(maxval),
                                   _ptr(workspace_buf), workspace_buf.numel(), _stream(stream))
    _check(rc, "spec_lm_head_argmax")


NOALLOC_MAX_ROWS = 8192


def spec_lm_head_argmax_noalloc(hidden, w_packed, V, argmax, maxval=None, stream=None):
    """spec_lm_head_argmax with no workspace: the library keeps its ticket and keys in
    a device array of its own (rows R <= NOALLOC_MAX_ROWS; calls on one GPU must not
    overlap in time)."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    _want(argmax, torch.int32, "argmax", 1)
    if maxval is not None:
        _want(maxval, torch.float32, "maxval", 1)
    R, H = hidden.shape
    if w_packed.numel() * 2 != lm_head_packed_bytes(V, H):
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {lm_head_packed_bytes(V, H)} "
                        f"for V={V} H={H}")
    _shape(argmax, (R,), "argmax")
    if maxval is not None:
        _shape(maxval, (R,), "maxval")
    rc = lib().spec_lm_head_argmax_noalloc(_ptr(hidden), _ptr(w_packed), R, H, V, _ptr(argmax), _ptr(maxval),
                                           _stream(stream))
    _check(rc, "spec_lm_head_argmax_noalloc")


def spec_greedy_accept(argmax, drafts, k, d2t, V, pos_in, pos_out, accept_len, n_emit, emit, next_tok,
                       seq_status, stream=None):
    """argmax [R], drafts [B,kmax], k [B], d2t [n] or None, pos_in/pos_out/accept_len/n_emit/next_tok/
    seq_status [B], emit [B,kmax+1] (int32)."""
    for t, n in ((argmax, "argmax"), (drafts, "drafts"), (k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"),
                 (accept_len, "accept_len"), (n_emit, "n_emit"), (emit, "emit"), (next_tok, "next_tok"),
                 (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    _want(drafts, torch.int32, "drafts", 2)
    B, kmax = drafts.shape
    R = argmax.shape[0]
    _shape(argmax, (R,), "argmax")
    _shape(emit, (B, kmax + 1), "emit")
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    rc = lib().spec_greedy_accept(_ptr(argmax), _ptr(drafts), kmax, _ptr(k), _ptr(d2t),
                                  0 if d2t is None else d2t.shape[0], V, B, R, _ptr(pos_in), _ptr(pos_out),
                                  _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok),
                                  _ptr(seq_status), _stream(stream))
    _check(rc, "spec_greedy_accept")


def spec_lm_head_argmax_accept(hidden, w_packed, V, argmax, maxval, drafts, k, d2t, pos_in, pos_out, accept_len,
                               n_emit, emit, next_tok, seq_status, workspace_buf=None, stream=None):
    """spec_lm_head_argmax then spec_greedy_accept on its argmax, in one call (same arguments
    and outputs as the two; the workspace as spec_lm_head_argmax's)."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    _want(argmax, torch.int32, "argmax", 1)
    if maxval is not None:
        _want(maxval, torch.float32, "maxval", 1)
    for t, n in ((drafts, "drafts"), (k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (emit, "emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    _want(drafts, torch.int32, "drafts", 2)
    R, H = hidden.shape
    B, kmax = drafts.shape
    if w_packed.numel() * 2 != lm_head_packed_bytes(V, H):
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {lm_head_packed_bytes(V, H)} "
                        f"for V={V} H={H}")
    _shape(argmax, (R,), "argmax")
    if maxval is not None:
        _shape(maxval, (R,), "maxval")
    _shape(emit, (B, kmax + 1), "emit")
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    if workspace_buf is None:
        workspace_buf = workspace(lm_head_argmax_workspace_bytes(R, H, V), hidden.device, zero=True)
    rc = lib().spec_lm_head_argmax_accept(_ptr(hidden), _ptr(w_packed), R, H, V, _ptr(argmax), _ptr(maxval),
                                          _ptr(drafts), kmax, _ptr(k), _ptr(d2t), 0 if d2t is None else d2t.shape[0],
                                          B, _ptr(pos_in), _ptr(pos_out), _ptr(accept_len), _ptr(n_emit), _ptr(emit),
                                          _ptr(next_tok), _ptr(seq_status), _ptr(workspace_buf),
                                          workspace_buf.numel(), _stream(stream))
    _check(rc, "spec_lm_head_argmax_accept")


def lm_head_sample_workspace_bytes(R, H, V) -> int:
    return lib().spec_lm_head_sample_workspace_bytes(R, H, V)


def spec_lm_head_sample(hidden, w_packed, V, temperature, q_tok, q_prob, row_ctr, seed, lse, z_supp, sample_p,
                        sample_res, workspace_buf=None, stream=None):
    """hidden [R,H] bf16, w_packed from spec_lm_head_pack; q_tok [R,NQ] int32 / q_prob [R,NQ] fp32
    (NQ may be 0: pass tensors of shape [R,0]); row_ctr [R,2] int32; outputs lse [R] fp32,
    z_supp [R,NQ] fp32, sample_p/sample_res [R] int32. A workspace_buf may hold anything."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    R, H = hidden.shape
    for t, n in ((q_tok, "q_tok"), (row_ctr, "row_ctr"), (sample_p, "sample_p"), (sample_res, "sample_res")):
        _want(t, torch.int32, n)
    for t, n in ((q_prob, "q_prob"), (lse, "lse"), (z_supp, "z_supp")):
        _want(t, torch.float32, n)
    NQ = q_tok.shape[1]
    _shape(q_tok, (R, NQ), "q_tok")
    _shape(q_prob, (R, NQ), "q_prob")
    _shape(z_supp, (R, NQ), "z_supp")
    _shape(row_ctr, (R, 2), "row_ctr")
    for t, n in ((lse, "lse"), (sample_p, "sample_p"), (sample_res, "sample_res")):
        _shape(t, (R,), n)
    if w_packed.numel() * 2 != lm_head_packed_bytes(V, H):
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {lm_head_packed_bytes(V, H)}")
    if workspace_buf is None:
        workspace_buf = workspace(lm_head_sample_workspace_bytes(R, H, V), hidden.device, zero=True)
    nz = lambda t: _ptr(t) if t.numel() else None
    rc = lib().spec_lm_head_sample(_ptr(hidden), _ptr(w_packed), R, H, V, float(temperature), nz(q_tok), nz(q_prob),
                                   NQ, _ptr(row_ctr), int(seed) & ((1 << 64) - 1), _ptr(lse), nz(z_supp),
                                   _ptr(sample_p), _ptr(sample_res), _ptr(workspace_buf), workspace_buf.numel(),
                                   _stream(stream))
    _check(rc, "spec_lm_head_sample")


def spec_sample_accept(drafts, k, d2t, V, q_tok, q_prob, lse, z_supp, sample_p, sample_res, row_ctr, seed, pos_in,
                       pos_out, accept_len, n_emit, emit, next_tok, seq_status, stream=None):
    """The speculative-sampling chain walk; drafts [B,kmax], the per-row arrays of
    spec_lm_head_sample, outputs as spec_greedy_accept."""
    for t, n in ((drafts, "drafts"), (k, "k"), (q_tok, "q_tok"), (sample_p, "sample_p"), (sample_res, "sample_res"),
                 (row_ctr, "row_ctr"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (emit, "emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    for t, n in ((q_prob, "q_prob"), (lse, "lse"), (z_supp, "z_supp")):
        _want(t, torch.float32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    _want(drafts, torch.int32, "drafts", 2)
    B, kmax = drafts.shape
    R = lse.shape[0]
    NQ = q_tok.shape[1]
    _shape(q_tok, (R, NQ), "q_tok")
    _shape(q_prob, (R, NQ), "q_prob")
    _shape(z_supp, (R, NQ), "z_supp")
    _shape(row_ctr, (R, 2), "row_ctr")
    _shape(emit, (B, kmax + 1), "emit")
    for t, n in ((sample_p, "sample_p"), (sample_res, "sample_res")):
        _shape(t, (R,), n)
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    nz = lambda t: _ptr(t) if t.numel() else None
    rc = lib().spec_sample_accept(nz(drafts), kmax, _ptr(k), _ptr(d2t), 0 if d2t is None else d2t.shape[0], V, B, R,
                                  nz(q_tok), nz(q_prob), NQ, _ptr(lse), nz(z_supp), _ptr(sample_p), _ptr(sample_res),
                                  _ptr(row_ctr), int(seed) & ((1 << 64) - 1), _ptr(pos_in), _ptr(pos_out),
                                  _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok), _ptr(seq_status),
                                  _stream(stream))
    _check(rc, "spec_sample_accept")


def spec_lm_head_sample_dense(hidden, w_packed, V, temperature, row_ctr, seed, lse, sample_p, z, workspace_buf=None,
                              stream=None):
    """The sampling pass for dense draft distributions: lse [R] fp32, sample_p [R] int32 (a
    draw from p of every row) and z [R,V] fp32 (logit / temperature of every entry). A
    workspace_buf (spec_lm_head_sample's size) may hold anything."""
    _want(hidden, torch.bfloat16, "hidden", 2)
    _want(w_packed, torch.bfloat16, "w_packed", 1)
    R, H = hidden.shape
    for t, n in ((row_ctr, "row_ctr"), (sample_p, "sample_p")):
        _want(t, torch.int32, n)
    for t, n in ((lse, "lse"), (z, "z")):
        _want(t, torch.float32, n)
    _shape(row_ctr, (R, 2), "row_ctr")
    _shape(z, (R, V), "z")
    for t, n in ((lse, "lse"), (sample_p, "sample_p")):
        _shape(t, (R,), n)
    if w_packed.numel() * 2 != lm_head_packed_bytes(V, H):
        raise SpecError(f"w_packed: {w_packed.numel() * 2} bytes, expected {lm_head_packed_bytes(V, H)}")
    if workspace_buf is None:
        workspace_buf = workspace(lm_head_sample_workspace_bytes(R, H, V), hidden.device, zero=True)
    rc = lib().spec_lm_head_sample_dense(_ptr(hidden), _ptr(w_packed), R, H, V, float(temperature), _ptr(row_ctr),
                                         int(seed) & ((1 << 64) - 1), _ptr(lse), _ptr(sample_p), _ptr(z),
                                         _ptr(workspace_buf), workspace_buf.numel(), _stream(stream))
    _check(rc, "spec_lm_head_sample_dense")


def sample_accept_dense_workspace_bytes(B) -> int:
    return lib().spec_sample_accept_dense_workspace_bytes(B)


def spec_sample_accept_dense(drafts, k, d2t, q, z, lse, sample_p, row_ctr, seed, pos_in, pos_out, accept_len, n_emit,
                             emit, next_tok, seq_status, workspace_buf=None, stream=None):
    """The chain walk with a dense draft distribution q [R,V] fp32 over the target
    vocabulary; z, lse and sample_p from spec_lm_head_sample_dense; outputs as
    spec_greedy_accept."""
    for t, n in ((drafts, "drafts"), (k, "k"), (sample_p, "sample_p"), (row_ctr, "row_ctr"), (pos_in, "pos_in"),
                 (pos_out, "pos_out"), (accept_len, "accept_len"), (n_emit, "n_emit"), (emit, "emit"),
                 (next_tok, "next_tok"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    for t, n in ((q, "q"), (z, "z"), (lse, "lse")):
        _want(t, torch.float32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    _want(drafts, torch.int32, "drafts", 2)
    _want(q, torch.float32, "q", 2)
    B, kmax = drafts.shape
    R, V = q.shape
    _shape(z, (R, V), "z")
    _shape(row_ctr, (R, 2), "row_ctr")
    _shape(emit, (B, kmax + 1), "emit")
    for t, n in ((lse, "lse"), (sample_p, "sample_p")):
        _shape(t, (R,), n)
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    if workspace_buf is None:
        workspace_buf = workspace(sample_accept_dense_workspace_bytes(B), q.device)
    rc = lib().spec_sample_accept_dense(_ptr(drafts) if drafts.numel() else None, kmax, _ptr(k), _ptr(d2t),
                                        0 if d2t is None else d2t.shape[0], V, B, R, _ptr(q), _ptr(z), _ptr(lse),
                                        _ptr(sample_p), _ptr(row_ctr), int(seed) & ((1 << 64) - 1), _ptr(pos_in),
                                        _ptr(pos_out), _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok),
                                        _ptr(seq_status), _ptr(workspace_buf), workspace_buf.numel(), _stream(stream))
    _check(rc, "spec_sample_accept_dense")


def spec_greedy_accept_stop(argmax, drafts, k, d2t, V, stop_ids, remaining, pos_in, pos_out, accept_len, n_emit,
                            emit, next_tok, done, seq_status, stream=None):
    """spec_greedy_accept with stop tokens (stop_ids [n_stop] int32 device tensor, n_stop <= 16)
    and an optional per-sequence limit remaining [B] (None: no limit); done [B] out."""
    for t, n in ((argmax, "argmax"), (drafts, "drafts"), (k, "k"), (stop_ids, "stop_ids"), (pos_in, "pos_in"),
                 (pos_out, "pos_out"), (accept_len, "accept_len"), (n_emit, "n_emit"), (emit, "emit"),
                 (next_tok, "next_tok"), (done, "done"), (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    if d2t is not None:
        _want(d2t, torch.int32, "d2t", 1)
    if remaining is not None:
        _want(remaining, torch.int32, "remaining", 1)
    _want(drafts, torch.int32, "drafts", 2)
    B, kmax = drafts.shape
    R = argmax.shape[0]
    _shape(emit, (B, kmax + 1), "emit")
    for t, n in ((k, "k"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (next_tok, "next_tok"), (done, "done"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    if remaining is not None:
        _shape(remaining, (B,), "remaining")
    n_stop = stop_ids.numel()
    rc = lib().spec_greedy_accept_stop(_ptr(argmax), _ptr(drafts) if drafts.numel() else None, kmax, _ptr(k),
                                       _ptr(d2t), 0 if d2t is None else d2t.shape[0], V, B, R,
                                       _ptr(stop_ids) if n_stop else None, n_stop, _ptr(remaining), _ptr(pos_in),
                                       _ptr(pos_out), _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok),
                                       _ptr(done), _ptr(seq_status), _stream(stream))
    _check(rc, "spec_greedy_accept_stop")


def spec_truncate_stop(stop_ids, remaining, pos_in, pos_out, accept_len, n_emit, emit, next_tok, done, seq_status,
                       path=None, stream=None):
    """The stop-token / limit rule applied in place to an acceptance walk's outputs
    (emit [B, kmax+1], the [B] scalars, and the tree walk's path [B, kmax] or None);
    stop_ids [n_stop] int32 device tensor (n_stop <= 16), remaining [B] or None; done [B] out."""
    for t, n in ((stop_ids, "stop_ids"), (pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"),
                 (n_emit, "n_emit"), (emit, "emit"), (next_tok, "next_tok"), (done, "done"),
                 (seq_status, "seq_status")):
        _want(t, torch.int32, n)
    _want(emit, torch.int32, "emit", 2)
    B, kmax = emit.shape[0], emit.shape[1] - 1
    for t, n in ((pos_in, "pos_in"), (pos_out, "pos_out"), (accept_len, "accept_len"), (n_emit, "n_emit"),
                 (next_tok, "next_tok"), (done, "done"), (seq_status, "seq_status")):
        _shape(t, (B,), n)
    if remaining is not None:
        _want(remaining, torch.int32, "remaining", 1)
        _shape(remaining, (B,), "remaining")
    if path is not None:
        _want(path, torch.int32, "path", 2)
        _shape(path, (B, kmax), "path")
    n_stop = stop_ids.numel()
    rc = lib().spec_truncate_stop(kmax, B, _ptr(stop_ids) if n_stop else None, n_stop, _ptr(remaining), _ptr(pos_in),
                                  _ptr(pos_out), _ptr(accept_len), _ptr(n_emit), _ptr(emit), _ptr(next_tok),
                                  _ptr(path) if path is not None and path.numel() else None, _ptr(done),
                                  _ptr(seq_status), _stream(stream))
    _check(rc, "spec_truncate_stop")


class KPolicy:
    """The library's adaptive draft-depth policy (spec_kpolicy_*), host side."""

    def __init__(self, kmin=1, kmax=6, prior_p=0.7, prior_n=8.0, draft_us=0.0, table=((1.0, 1.0),)):
        rows = (ctypes.c_double * len(table))(*[float(r) for r, _ in table])
        us = (ctypes.c_double * len(table))(*[float(t) for _, t in table])
        self.st = _KPolicyStruct()
        _check(lib().spec_kpolicy_init(ctypes.byref(self.st), kmin, kmax, prior_p, prior_n, draft_us, rows, us,
                                       len(table)), "spec_kpolicy_init")

    def p(self, j):
        return lib().spec_kpolicy_accept_prob(ctypes.byref(self.st), j)

    def verify_cost(self, rows):
        return lib().spec_kpolicy_verify_cost(ctypes.byref(self.st), float(rows))

    def expected_tokens(self, k):
        return lib().spec_kpolicy_expected_tokens(ctypes.byref(self.st), k)

    def choose(self, B, row_cap=0):
        return lib().spec_kpolicy_choose(ctypes.byref(self.st), B, row_cap)

    def update(self, k, accepted):
        lib().spec_kpolicy_update(ctypes.byref(self.st), k, accepted)

    def update_batch(self, k, accept_len):
        """k, accept_len: host int32 arrays [B] (e.g. the accept call's outputs, copied back)."""
        import numpy as np
        k = np.ascontiguousarray(k, np.int32)
        a = np.ascontiguousarray(accept_len, np.int32)
        _check(lib().spec_kpolicy_update_batch(ctypes.byref(self.st), k.ctypes.data_as(ctypes.c_void_p),
                                               a.ctypes.data_as(ctypes.c_void_p), len(k)), "spec_kpolicy_update_batch")


def spec_delta_verify_rollback(mode, q, k, v, a, b, q_scale, state, rec, L, o=None, stream=None):
    """q,k [B,T,Hd,dk], v [B,T,Hd,dv] bf16; a,b [B,T,Hd] fp32; state [B,Hd,dv,dk] fp32;
    rec [B,T,Hd,dv,dk] fp32 (None in modes VERIFY/RESCAN); L [B] int32 (None in modes
    RECORD/VERIFY); o [B,T,Hd,dv] bf16 or None."""
    _want(state, torch.float32, "state", 4)
    scans = mode != DELTA_ROLLBACK
    if scans:
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _want(t, torch.bfloat16, n, 4)
        B, T, Hd, dk = q.shape
        dv = v.shape[3]
    else:
        _want(rec, torch.float32, "rec", 5)
        B, T, Hd, dv, dk = rec.shape
    _shape(state, (B, Hd, dv, dk), "state")
    if rec is not None:
        _want(rec, torch.float32, "rec", 5)
        _shape(rec, (B, T, Hd, dv, dk), "rec")
    elif mode in (DELTA_RECORD, DELTA_ROLLBACK, DELTA_BOTH):
        raise SpecError(f"spec_delta_verify_rollback: rec required in mode {mode}")
    if scans:
        _want(a, torch.float32, "a", 3)
        _want(b, torch.float32, "b", 3)
        _shape(q, (B, T, Hd, dk), "q")
        _shape(k, (B, T, Hd, dk), "k")
        _shape(v, (B, T, Hd, dv), "v")
        _shape(a, (B, T, Hd), "a")
        _shape(b, (B, T, Hd), "b")
    if L is not None:
        _want(L, torch.int32, "L", 1)
        _shape(L, (B,), "L")
    if o is not None:
        _want(o, torch.bfloat16, "o", 4)
        _shape(o, (B, T, Hd, dv), "o")
    rc = lib().spec_delta_verify_rollback(mode, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), q_scale,
                                          _ptr(state), _ptr(rec), _ptr(L), B, T, Hd, dk, dv, _ptr(o),
                                          _stream(stream))
    _check(rc, "spec_delta_verify_rollback")
