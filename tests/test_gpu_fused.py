"""spec_lm_head_argmax_accept against spec_lm_head_argmax followed by spec_greedy_accept:
the same bytes for every output and status, on the fused path (R <= 96 with the full
workspace) and on the general one (more rows, or a workspace without the key rows),
with ragged k, a draft vocabulary map, flagged sequences and an undefined packing.
Every call leaves its workspace zero. At the b16k4 sizes the acceptance is also
checked against the oracle's walk on the same greedy tokens."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

OUT_NAMES = ("argmax", "maxval", "pos_out", "accept_len", "n_emit", "emit", "next_tok", "seq_status")


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _run(gdv, fused, h, wp, V, drafts, k, d2t, pos, ws_bytes=None):
    dev = h.device
    R, H = h.shape
    B, kmax = drafts.shape
    i32 = lambda shape: torch.full(shape, -7, dtype=torch.int32, device=dev)
    o = {"argmax": i32((R,)), "maxval": torch.full((R,), float("nan"), device=dev), "pos_out": i32((B,)),
         "accept_len": i32((B,)), "n_emit": i32((B,)), "emit": i32((B, kmax + 1)), "next_tok": i32((B,)),
         "seq_status": i32((B,))}
    ws = gdv.workspace(ws_bytes or gdv.lm_head_argmax_workspace_bytes(R, H, V), dev, zero=True)
    acc = (drafts, k, d2t, pos, o["pos_out"], o["accept_len"], o["n_emit"], o["emit"], o["next_tok"],
           o["seq_status"])
    if fused:
        gdv.spec_lm_head_argmax_accept(h, wp, V, o["argmax"], o["maxval"], *acc, workspace_buf=ws)
    else:
        gdv.spec_lm_head_argmax(h, wp, V, o["argmax"], o["maxval"], workspace_buf=ws)
        gdv.spec_greedy_accept(o["argmax"], drafts, k, d2t, V, *acc[3:])
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0, "workspace not left zero"
    return {n: o[n].cpu() for n in OUT_NAMES}


def _same(a, b, what):
    for n in OUT_NAMES:
        x, y = a[n], b[n]
        if n == "maxval":
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{what}: {n} differs"


# name, B, k range, kmax, H, V, with d2t, special
CASES = [
    ("one_row", 1, (0, 0), 0, 256, 1000, False, None),
    ("b1k3", 1, (3, 3), 3, 256, 1000, False, None),
    ("b16k4", 16, (4, 4), 4, 512, 5000, False, None),
    ("ragged_d2t", 12, (0, 7), 7, 256, 20000, True, None),
    ("r96", 24, (3, 3), 3, 256, 3000, False, None),
    ("r97_general", 97, (0, 0), 0, 256, 3000, False, None),
    ("long_chain", 1, (70, 70), 80, 256, 2000, False, None),
    ("two_long", 2, (40, 47), 47, 256, 20000, True, None),
    ("small_ws", 16, (4, 4), 4, 256, 5000, False, "small_ws"),
    ("bad_pos", 6, (2, 5), 5, 256, 3000, False, "bad_pos"),
    ("k_over_kmax", 6, (2, 5), 4, 256, 3000, False, "k_over_kmax"),
    ("bad_packing", 5, (1, 4), 4, 256, 3000, False, "bad_packing"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_lm_head_then_accept(dev, case):
    import greedy_draft_verify_amd as gdv
    name, B, (k_lo, k_hi), kmax, H, V, with_d2t, special = case
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k = rng.integers(k_lo, k_hi + 1, B).astype(np.int32)
    if special == "k_over_kmax":
        k[2] = kmax + 1
    R = int((k + 1).sum()) + (1 if special == "bad_packing" else 0)
    w = torch.from_numpy((rng.standard_normal((V, H)) / math.sqrt(H)).astype(np.float32)).to(torch.bfloat16)
    wp = gdv.spec_lm_head_pack(w.to(dev))
    h = torch.from_numpy(rng.standard_normal((R, H)).astype(np.float32)).to(torch.bfloat16).to(dev)
    # the greedy tokens, then drafts that follow them with probability 0.6
    g = torch.empty(R, dtype=torch.int32, device=dev)
    gdv.spec_lm_head_argmax(h, wp, V, g)
    g = g.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(k + 1)])
    d2t_np = None
    if with_d2t:
        n_d = 4096
        d2t_np = rng.integers(0, V, n_d).astype(np.int32)
        d2t_np[: len(np.unique(g))] = np.unique(g)
        rng.shuffle(d2t_np)
        inv = {int(t): i for i, t in enumerate(d2t_np)}
    drafts = np.zeros((B, max(kmax, 1) if kmax else 0), np.int32)
    for s in range(B):
        for j in range(min(int(k[s]), kmax)):
            r = off[s] + j
            keep = rng.random() < 0.6 and r < R
            tgt = int(g[r]) if keep else int(rng.integers(0, V))
            drafts[s, j] = inv.get(tgt, 0) if with_d2t else tgt
    pos = rng.integers(0, 5000, B).astype(np.int32)
    if special == "bad_pos":
        pos[1] = -3
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d2t = t(d2t_np) if with_d2t else None
    ws_bytes = 256 + 8 * R if special == "small_ws" else None
    a = _run(gdv, True, h, wp, V, t(drafts), t(k), d2t, t(pos), ws_bytes)
    b = _run(gdv, False, h, wp, V, t(drafts), t(k), d2t, t(pos), ws_bytes)
    _same(a, b, name)
    st = a["seq_status"].numpy()
    if special is None or special == "small_ws":
        assert (st == 0).all()
        assert (a["accept_len"].numpy() >= 0).all()
    elif special == "bad_packing":
        assert (st != 0).all()
    elif special == "bad_pos":
        assert st[1] != 0 and (st[(k <= kmax) & (pos >= 0)] == 0).all()
    else:
        assert ((st != 0) == (k > kmax)).all() and st[2] != 0


def test_fused_b16k4_full_size(dev):
    """The benchmark's configuration (80 rows, H = 4096, V = 151936): the fused call gives
    the separate calls' bytes, its acceptance equals the oracle's walk on its greedy
    tokens, and 10 calls in a row give the same bytes."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16k4", seed=0, device=dev)
    wp = gdv.spec_lm_head_pack(x.w)
    x.w = None
    V = x.wl.V
    g = torch.empty(x.R, dtype=torch.int32, device=dev)
    gdv.spec_lm_head_argmax(x.hidden, wp, V, g)
    g0 = g.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    drafts_np = synth.make_drafts(x.wl, x.k, [g0[off[s]:off[s] + x.k[s]] for s in range(len(x.pos))], seed=0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    drafts, k, pos = t(drafts_np), t(x.k), t(x.pos)
    a = _run(gdv, True, x.hidden, wp, V, drafts, k, None, pos)
    b = _run(gdv, False, x.hidden, wp, V, drafts, k, None, pos)
    _same(a, b, "b16k4")
    B, kmax = drafts_np.shape
    ref = oracle.greedy_accept(a["argmax"].numpy(), drafts_np, kmax, x.k, None, 0, V, B, x.R, x.pos)
    assert (a["seq_status"].numpy() == 0).all()
    for n in ("pos_out", "accept_len", "n_emit", "emit", "next_tok"):
        assert np.array_equal(a[n].numpy(), ref[n]), n
    for _ in range(10):
        _same(_run(gdv, True, x.hidden, wp, V, drafts, k, None, pos), a, "b16k4 repeat")
