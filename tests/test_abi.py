"""The C ABI library: it loads, exports every symbol the header declares, and its
host-side argument checks reject bad calls before anything reaches a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import greedy_draft_verify_amd as gdv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"spec_verify_attn", "spec_lm_head_argmax", "spec_greedy_accept",
            "spec_delta_verify_rollback", "spec_verify_attn_tree", "spec_tree_accept",
            "spec_kv_compact", "spec_lm_head_sample", "spec_sample_accept",
            "spec_greedy_accept_stop"} <= set(names)
    lib = gdv.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gdv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spec_\w+)", out))
    assert set(names) <= exported
    assert set(gdv.EXPORTED) == set(names)


def test_version_and_split_rule():
    assert gdv.version() >= 1
    # capacity-derived split: power of two >= 256 with <= 64 splits, capped at 2048
    assert gdv.attn_split_tokens(32) == 256
    assert gdv.attn_split_tokens(260) == 256
    assert gdv.attn_split_tokens(2052) == 1024
    assert gdv.attn_split_tokens(8196) == 2048


def _vp(x=0x1000):
    return ctypes.c_void_p(x)


def test_host_argument_checks():
    L = gdv.lib()
    p = _vp()
    # D outside {64,128,256}
    rc = L.spec_verify_attn(p, p, p, p, p, 10, p, 4, p, p, 3, 1, 4, 4, 1, 100, 0.1, 0, p, p, 1 << 30, p, None)
    assert rc == -1 and b"D=100" in L.spec_last_error()
    # Hq % Hkv != 0
    rc = L.spec_verify_attn(p, p, p, p, p, 10, p, 4, p, p, 3, 1, 4, 6, 4, 128, 0.1, 0, p, p, 1 << 30, p, None)
    assert rc == -1
    # split not a multiple of 64
    rc = L.spec_verify_attn(p, p, p, p, p, 10, p, 4, p, p, 3, 1, 4, 4, 1, 64, 0.1, 100, p, p, 1 << 30, p, None)
    assert rc == -1
    # misaligned pointer
    rc = L.spec_verify_attn(_vp(0x1002), p, p, p, p, 10, p, 4, p, p, 3, 1, 4, 4, 1, 64, 0.1, 0, p, p, 1 << 30, p, None)
    assert rc == -1 and b"aligned" in L.spec_last_error()
    # kmax past the draft limit (127)
    rc = L.spec_verify_attn(p, p, p, p, p, 10, p, 4, p, p, 128, 1, 4, 16, 1, 64, 0.1, 0, p, p, 1 << 30, p, None)
    assert rc == -1 and b"kmax" in L.spec_last_error()
    # workspace too small
    rc = L.spec_verify_attn(p, p, p, p, p, 10, p, 4, p, p, 3, 1, 4, 4, 1, 64, 0.1, 0, p, p, 16, p, None)
    assert rc == -4
    need = L.spec_verify_attn_workspace_bytes(1, 4, 4, 1, 64, 4, 0)
    assert need > 0
    # lm_head: H not a multiple of 128, workspace
    assert L.spec_lm_head_argmax(p, p, 4, 100, 1000, p, None, p, 1 << 30, None) == -1
    assert L.spec_lm_head_argmax(p, p, 4, 256, 1000, p, None, p, 8, None) == -4
    assert L.spec_lm_head_argmax_workspace_bytes(4, 256, 1000) >= 4 * 8 * 8
    assert L.spec_lm_head_pack(p, 1000, 128, p, None) == -1
    assert L.spec_lm_head_packed_bytes(1000, 256) == 1024 * 256 * 2
    # accept: B out of range, null pointers
    assert L.spec_greedy_accept(p, p, 3, p, None, 0, 100, 0, 4, p, p, p, p, p, p, p, None) == -1
    assert L.spec_greedy_accept(p, None, 3, p, None, 0, 100, 1, 4, p, p, p, p, p, p, p, None) == -1
    # delta: mode, dims, missing L
    assert L.spec_delta_verify_rollback(6, p, p, p, p, p, 1.0, p, p, p, 1, 5, 1, 128, 128, None, None) == -1
    assert L.spec_delta_verify_rollback(5, p, p, p, p, p, 1.0, p, None, None, 1, 5, 1, 128, 128, None, None) == -1
    assert L.spec_delta_verify_rollback(4, None, p, p, p, p, 1.0, p, None, None, 1, 5, 1, 128, 128, None, None) == -1
    assert L.spec_delta_verify_rollback(1, p, p, p, p, p, 1.0, p, None, None, 1, 5, 1, 128, 128, None, None) == -1
    assert L.spec_delta_verify_rollback(1, p, p, p, p, p, 1.0, p, p, None, 1, 5, 1, 64, 128, None, None) == -1
    assert L.spec_delta_verify_rollback(2, p, p, p, p, p, 1.0, p, p, None, 1, 5, 1, 128, 128, None, None) == -1
    assert L.spec_last_error() != b""
    # tree calls
    need = L.spec_verify_attn_tree_workspace_bytes(2, 8, 4, 1, 64, 4, 0, 3)
    # the ancestor masks live in LDS, so a tree call needs the chain call's workspace
    assert need == L.spec_verify_attn_workspace_bytes(2, 8, 4, 1, 64, 4, 0) > 0
    assert L.spec_verify_attn_tree_workspace_bytes(2, 8, 4, 1, 64, 4, 0, -1) == 0
    tree = lambda parent, kmax, ws: L.spec_verify_attn_tree(p, p, p, p, p, 10, p, 4, p, p, parent, kmax, 2, 8, 4, 1,
                                                            64, 0.1, 0, p, p, ws, p, None)
    assert tree(None, 3, 1 << 30) == -1 and b"parent" in L.spec_last_error()
    assert tree(p, 128, 1 << 30) == -1 and b"kmax" in L.spec_last_error()
    assert tree(p, 3, need - 1) == -4
    # the LDS limit: at D = 256 a tree call holds K and V of kmax new rows beside the tile
    tree256 = lambda kmax: L.spec_verify_attn_tree(p, p, p, p, p, 10, p, 4, p, p, p, kmax, 2, 8, 1, 1, 256, 0.1, 0,
                                                   p, p, 1 << 30, p, None)
    assert tree256(94) == -1 and b"LDS" in L.spec_last_error()
    acc = lambda kmax, parent, path: L.spec_tree_accept(p, p, kmax, p, parent, None, 0, 100, 2, 8, p, p, p, p, p,
                                                        p, path, p, None)
    assert acc(128, p, p) == -1 and b"kmax" in L.spec_last_error()
    assert acc(3, None, p) == -1 and b"null" in L.spec_last_error()
    assert acc(3, p, None) == -1
    cmp = lambda D, Hkv, kmax: L.spec_kv_compact(p, p, 10, p, 4, p, p, p, kmax, 2, Hkv, D, p, None)
    assert cmp(100, 1, 3) == -1 and b"D=100" in L.spec_last_error()
    assert cmp(64, 0, 3) == -1 and cmp(64, 1, 128) == -1
    assert L.spec_kv_compact(_vp(0x1002), p, 10, p, 4, p, p, p, 3, 2, 1, 64, p, None) == -1
    assert b"aligned" in L.spec_last_error()
    # sampling calls
    need = L.spec_lm_head_sample_workspace_bytes(8, 256, 1000)
    assert need >= 256 + 8 * 8 + 8 * 8 * 8      # keys + (max, sum) per (row, 128-entry group)
    smp = lambda T, NQ, ws: L.spec_lm_head_sample(p, p, 8, 256, 1000, T, p, p, NQ, p, 1, p, p, p, p, p, ws, None)
    assert smp(0.0, 1, 1 << 30) == -1 and b"temperature" in L.spec_last_error()
    assert smp(float("inf"), 1, 1 << 30) == -1
    assert smp(1.0, 9, 1 << 30) == -1 and b"NQ" in L.spec_last_error()
    assert smp(1.0, 1, need - 1) == -4
    acc = lambda B, NQ: L.spec_sample_accept(p, 3, p, None, 0, 100, B, 8, p, p, NQ, p, p, p, p, p, 1, p, p, p, p, p,
                                             p, p, None)
    assert acc(0, 1) == -1 and acc(2, 9) == -1
    assert L.spec_sample_accept(None, 3, p, None, 0, 100, 2, 8, p, p, 1, p, p, p, p, p, 1, p, p, p, p, p, p, p,
                                None) == -1
    stop = lambda n_stop, stops, done: L.spec_greedy_accept_stop(p, p, 3, p, None, 0, 100, 2, 8, stops, n_stop, None,
                                                                 p, p, p, p, p, p, done, p, None)
    assert stop(17, p, p) == -1 and b"n_stop" in L.spec_last_error()
    assert stop(2, None, p) == -1 and stop(2, p, None) == -1


def test_product_path_does_not_touch_the_oracle():
    """The package never imports or links the oracle."""
    pkg = os.path.join(ROOT, "greedy_draft_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|oracle\.(so|h|c)\b", src, re.M), f
    out = subprocess.run(["ldd", gdv.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out


def test_fused_argmax_accept_checks_before_launching():
    """spec_lm_head_argmax_accept refuses bad acceptance or lm_head arguments with the
    codes of the two calls it stands for (host checks only: fake pointers never reach
    a kernel)."""
    L = gdv.lib()
    p = _vp()
    args = lambda B, kmax, H, ws: (p, p, 4, H, 1000, p, None, p, kmax, p, None, 0, B, p, p, p, p, p, p, p, p, ws,
                                   None)
    assert L.spec_lm_head_argmax_accept(*args(0, 3, 256, 1 << 30)) == -1          # B < 1
    assert b"B=0" in L.spec_last_error()
    assert L.spec_lm_head_argmax_accept(*args(1, 1025, 256, 1 << 30)) == -1       # kmax > 1024
    assert L.spec_lm_head_argmax_accept(*args(1, 3, 100, 1 << 30)) == -1         # H not a multiple of 256
    assert L.spec_lm_head_argmax_accept(*args(1, 3, 256, 8)) == -4                # workspace too small
    # a null required pointer of the acceptance
    assert L.spec_lm_head_argmax_accept(p, p, 4, 256, 1000, p, None, p, 3, None, None, 0, 1, p, p, p, p, p, p, p,
                                        p, 1 << 30, None) == -1
