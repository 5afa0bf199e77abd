"""The verify step captured as a HIP graph and replayed gives the eager step's bytes.

The benchmark times graph replays of spec_verify_attn -> spec_lm_head_argmax_accept
(the lm_head and the acceptance as one call; the two calls in turn give the same
bytes). This test captures that step, and the one with the two calls, for the b16k4 workload (the
benchmark's configuration) and for a ragged batch, replays it several times with
eager work and host synchronisations between the replays, and checks every output
of every replay against the eager step byte for byte (the step appends the same
K/V at the same slots each time, so replays are idempotent).
"""
import numpy as np
import pytest
import torch

from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "two_calls"])
@pytest.mark.parametrize("name", ["b16k4", "ragged"])
def test_graph_replay_matches_eager(name, fused):
    import bench
    dev = torch.device("cuda:0")
    x = synth.make_verify_inputs(name, seed=3, device=dev)
    step = bench.VerifyStep(x, dev)
    x.w = None
    step.lm_head()
    torch.cuda.synchronize()
    g0 = step.argmax.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    true_next = [g0[off[s]:off[s] + x.k[s]] for s in range(len(x.pos))]
    step.drafts = bench.i32(synth.make_drafts(x.wl, x.k, true_next, seed=3, d2t=x.d2t), dev)

    def run():
        step.attn()
        if fused:
            step.lm_head_accept()
        else:
            step.lm_head()
            step.accept()

    run()
    torch.cuda.synchronize()
    ref = step.outputs()
    assert (ref[1].cpu() == 0).all() and (ref[-1].cpu() == 0).all()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for t in (step.attn_out, step.argmax, step.maxval, step.acc_len, step.emit, step.next_tok):
            t.view(torch.uint8).fill_(0xA5)          # stale bytes a replay must overwrite
        graph.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"
        run()                                          # the program's own eager work between replays
        torch.cuda.synchronize()


def _replays_match(run, outputs, reps=4):
    """Captures run() as a graph; every replay (with stale output bytes before it and
    eager work after it) must give the eager bytes."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    for rep in range(reps):
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outputs)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: output {i} differs"
        run()
        torch.cuda.synchronize()


def test_graph_replay_tree_step():
    """Tree step (spec_verify_attn_tree -> spec_lm_head_argmax -> spec_tree_accept ->
    spec_kv_compact) on the 16-node tree workload: the append rewrites every node's slot,
    so a step after a compaction sees the same pool and the replays are idempotent."""
    import greedy_draft_verify_amd as gdv
    import bench
    dev = torch.device("cuda:0")
    x = synth.make_verify_inputs("b16tree", seed=1, device=dev, with_lm_head=False)
    wl = x.wl
    B, R, kmax = len(x.pos), x.R, wl.kmax
    hidden = synth.normal_bf16((R, 256), 1.0, 1, "tiny", "extra", dev)
    w = synth.normal_bf16((1000, 256), 1 / 16, 1, "tiny", "w", dev)
    wp = gdv.spec_lm_head_pack(w)
    parent_np = synth.make_parents(x.k, 1, wl.name, "trie")
    parent = bench.i32(parent_np, dev)
    pt, pos, k = bench.i32(x.page_table, dev), bench.i32(x.pos, dev), bench.i32(x.k, dev)
    out = torch.empty((R, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    am = torch.empty(R, dtype=torch.int32, device=dev)
    lm_ws = gdv.workspace(gdv.lm_head_argmax_workspace_bytes(R, 256, 1000), dev, zero=True)
    gdv.spec_lm_head_argmax(hidden, wp, 1000, am, None, workspace_buf=lm_ws)
    torch.cuda.synchronize()
    g0 = am.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    tw = synth.VerifyWorkload("tw", B=B, k=kmax, k_lo=kmax, k_hi=kmax, ctx_lo=0, ctx_hi=0, Hq=1, Hkv=1, D=64, H=1,
                              V=1000, max_pages=1)
    drafts = bench.i32(synth.make_tree_drafts(tw, x.k, parent_np, [g0[off[s]:off[s + 1]] for s in range(B)], 1), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, ast = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)
    path = torch.empty((B, kmax), dtype=torch.int32, device=dev)
    cst = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = gdv.workspace(gdv.verify_attn_tree_workspace_bytes(B, R, wl.Hq, wl.Hkv, wl.D, x.page_table.shape[1], kmax),
                       dev)

    def run():
        gdv.spec_verify_attn_tree(x.q, x.k_new, x.v_new, x.k_pool, x.v_pool, pt, pos, k, parent, x.scale, out, st,
                                  workspace_buf=ws)
        gdv.spec_lm_head_argmax(hidden, wp, 1000, am, None, workspace_buf=lm_ws)
        gdv.spec_tree_accept(am, drafts, k, parent, None, 1000, pos, pos_out, acc, ne, emit, nt, path, ast)
        cst.zero_()
        gdv.spec_kv_compact(x.k_pool, x.v_pool, pt, pos, path, acc, cst)

    _replays_match(run, [out, am, acc, emit, path, pos_out, st, cst])
    assert (st.cpu() == 0).all() and (cst.cpu() == 0).all() and acc.cpu().numpy().max() >= 1


def test_graph_replay_sampling_step():
    """Sampling step (spec_verify_attn -> spec_lm_head_sample -> spec_sample_accept) on the
    b16k4 shapes with a small vocabulary: the sample workspace's keys are reset by every
    call, so replays give the eager bytes."""
    import greedy_draft_verify_amd as gdv
    import bench
    dev = torch.device("cuda:0")
    x = synth.make_verify_inputs("b16k4", seed=2, device=dev, with_lm_head=False)
    B, R, kmax, V, H = len(x.pos), x.R, x.wl.kmax, 3000, 512
    hidden = synth.normal_bf16((R, H), 1.0, 2, "tiny", "extra", dev)
    w = synth.normal_bf16((V, H), 0.2, 2, "tiny", "w", dev)
    wp = gdv.spec_lm_head_pack(w)
    step = bench.VerifyStep(x, dev, w_packed=wp)
    rng = np.random.default_rng(4)
    drafts_np = rng.integers(0, V, (B, kmax)).astype(np.int32)
    step.drafts = bench.i32(drafts_np, dev)
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    q_tok = np.full((R, 2), -1, np.int32)
    q_prob = np.zeros((R, 2), np.float32)
    for s in range(B):
        for j in range(x.k[s]):
            q_tok[off[s] + j] = [drafts_np[s, j], rng.integers(0, V)]
            q_prob[off[s] + j] = [0.6, 0.4]
    q_tok_d, q_prob_d = bench.i32(q_tok, dev), torch.from_numpy(q_prob).to(dev)
    row_ctr = bench.i32(np.stack([np.arange(R), np.zeros(R)], 1), dev)
    lse = torch.empty(R, device=dev)
    z = torch.empty((R, 2), device=dev)
    sp = torch.empty(R, dtype=torch.int32, device=dev)
    sr = torch.empty(R, dtype=torch.int32, device=dev)
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, H, V), dev, zero=True)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, sst = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)

    def run():
        step.attn()
        gdv.spec_lm_head_sample(hidden, wp, V, 0.7, q_tok_d, q_prob_d, row_ctr, 99, lse, z, sp, sr, workspace_buf=ws)
        gdv.spec_sample_accept(step.drafts, step.k, None, V, q_tok_d, q_prob_d, lse, z, sp, sr, row_ctr, 99, step.pos,
                               pos_out, acc, ne, emit, nt, sst)

    _replays_match(run, [step.attn_out, lse, z, sp, sr, acc, emit, pos_out, sst])
    assert (sst.cpu() == 0).all()


def test_graph_replay_dense_sampling():
    """Dense-draft sampling (spec_lm_head_sample_dense -> spec_sample_accept_dense) captured
    and replayed: the walk initialises its workspace on every call, the sample pass leaves
    its own zero, so replays give the eager bytes."""
    import greedy_draft_verify_amd as gdv
    dev = torch.device("cuda:0")
    B, kmax, V, H = 16, 4, 3000, 512
    rng = np.random.default_rng(8)
    k = rng.integers(0, kmax + 1, B).astype(np.int32)
    R = int((k + 1).sum())
    hidden = synth.normal_bf16((R, H), 1.0, 3, "tiny", "extra", dev)
    w = synth.normal_bf16((V, H), 0.2, 3, "tiny", "w", dev)
    wp = gdv.spec_lm_head_pack(w)
    q = torch.softmax(torch.randn((R, V), generator=torch.Generator().manual_seed(5)), dim=1).to(dev)
    drafts = torch.multinomial(q[:B].cpu(), kmax, replacement=True).to(torch.int32)
    # each draft drawn from its own row's q
    off = np.concatenate([[0], np.cumsum(k + 1)])
    qc = q.cpu()
    for s in range(B):
        for j in range(k[s]):
            drafts[s, j] = int(torch.multinomial(qc[off[s] + j], 1))
    drafts = drafts.to(dev)
    kk = torch.from_numpy(k).to(dev)
    row_ctr = torch.from_numpy(np.stack([np.arange(R), np.full(R, 4)], 1).astype(np.int32)).to(dev)
    pos = torch.from_numpy(rng.integers(0, 900, B).astype(np.int32)).to(dev)
    lse = torch.empty(R, device=dev)
    sp = torch.empty(R, dtype=torch.int32, device=dev)
    z = torch.empty((R, V), device=dev)
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, H, V), dev, zero=True)
    wsd = gdv.workspace(gdv.sample_accept_dense_workspace_bytes(B), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, sst = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)

    def run():
        gdv.spec_lm_head_sample_dense(hidden, wp, V, 0.9, row_ctr, 123, lse, sp, z, workspace_buf=ws)
        gdv.spec_sample_accept_dense(drafts, kk, None, q, z, lse, sp, row_ctr, 123, pos, pos_out, acc, ne, emit, nt,
                                     sst, workspace_buf=wsd)

    _replays_match(run, [lse, sp, z, acc, emit, pos_out, sst])
    assert (sst.cpu() == 0).all()
