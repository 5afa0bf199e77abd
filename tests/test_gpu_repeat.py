"""Back-to-back calls give identical bytes.

A race between the waves of a workgroup (or between workgroups) can change a result
only now and then, by amounts far inside the oracle's tolerance; repeating a call on
device-resident inputs, as a decode loop does, and comparing every call's bytes with
the first catches such a race where the parity tests cannot. The verify step itself
(attention, lm_head, greedy walk) is repeated this way in tests/test_gpu_graph.py;
this file covers the tree step, the sampling passes and walks and the DeltaNet modes
at the benchmark's sizes.
"""
import numpy as np
import pytest
import torch

from greedy_draft_verify_amd import synth
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

REPS = 20


@pytest.fixture(scope="module")
def dev():
    import greedy_draft_verify_amd as gdv
    gdv.lib()
    return torch.device("cuda:0")


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


def _repeat(fn, outs, what):
    """Runs fn REPS times; after each call every tensor in outs must equal its first copy."""
    first = None
    for rep in range(REPS):
        fn()
        torch.cuda.synchronize()
        cur = [t.clone() for t in outs]
        if first is None:
            first = cur
            continue
        for j, (a, b) in enumerate(zip(first, cur)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: output {j} differs on call {rep}"


def test_tree_step_repeats(dev):
    """spec_verify_attn_tree (with its append), spec_tree_accept and spec_kv_compact on
    b16tree, each call on fresh copies of the pool."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16tree", seed=1, device=dev, with_lm_head=False)
    wl = x.wl
    B, R = len(x.pos), x.R
    parent = _i32(synth.make_parents(x.k, 1, "b16tree", "trie"), dev)
    pt, pos, k = _i32(x.page_table, dev), _i32(x.pos, dev), _i32(x.k, dev)
    out = torch.empty((R, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    kp, vp = x.k_pool.clone(), x.v_pool.clone()

    def attn():
        kp.copy_(x.k_pool)
        vp.copy_(x.v_pool)
        gdv.spec_verify_attn_tree(x.q, x.k_new, x.v_new, kp, vp, pt, pos, k, parent, x.scale, out, st)

    print("[repeat] tree attention", flush=True)
    _repeat(attn, [out, st, kp, vp], "tree attention")
    # the walk on random greedy tokens, then the compaction of the accepted paths
    rng = np.random.default_rng(1)
    g = _i32(rng.integers(0, 50, R), dev)
    drafts = _i32(rng.integers(0, 50, (B, wl.kmax)), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st2 = e(), e(), e(), e(), e()
    emit = torch.empty((B, wl.kmax + 1), dtype=torch.int32, device=dev)
    path = torch.empty((B, wl.kmax), dtype=torch.int32, device=dev)
    print("[repeat] tree accept", flush=True)
    _repeat(lambda: gdv.spec_tree_accept(g, drafts, k, parent, None, 50, pos, pos_out, acc, ne, emit, nt, path, st2),
            [pos_out, acc, ne, nt, st2, emit, path], "tree accept")
    cst = e()

    def compact():
        kp.copy_(x.k_pool)
        vp.copy_(x.v_pool)
        cst.zero_()
        gdv.spec_kv_compact(kp, vp, pt, pos, path, acc, cst)

    print("[repeat] kv compact", flush=True)
    _repeat(compact, [kp, vp, cst], "kv compact")


def test_sampling_passes_repeat(dev):
    """The sampling lm_head (sparse supports) and its walk, and the dense pass and walk,
    on the b16k4 rows."""
    import greedy_draft_verify_amd as gdv
    x = synth.make_verify_inputs("b16k4", seed=2, device=dev)
    R, V, B = x.R, x.wl.V, len(x.pos)
    kmax = x.wl.kmax
    wp = gdv.spec_lm_head_pack(x.w)
    x.w = None
    torch.cuda.empty_cache()
    rng = np.random.default_rng(2)
    NQ = 4
    q_tok = _i32(rng.integers(0, V, (R, NQ)), dev)
    qp = rng.uniform(0.1, 1.0, (R, NQ))
    q_prob = torch.from_numpy((qp / qp.sum(1, keepdims=True)).astype(np.float32)).to(dev)
    row_ctr = _i32(np.stack([np.arange(R) + 7, np.zeros(R)], 1), dev)
    lse = torch.empty(R, device=dev)
    z = torch.empty((R, NQ), device=dev)
    sp = torch.empty(R, dtype=torch.int32, device=dev)
    sr = torch.empty(R, dtype=torch.int32, device=dev)
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, x.wl.H, V), dev, zero=True)
    print("[repeat] sampling lm_head", flush=True)
    _repeat(lambda: gdv.spec_lm_head_sample(x.hidden, wp, V, 0.9, q_tok, q_prob, row_ctr, 11, lse, z, sp, sr,
                                            workspace_buf=ws), [lse, z, sp, sr], "sampling lm_head")
    k = _i32(x.k, dev)
    pos = _i32(x.pos, dev)
    drafts = _i32(rng.integers(0, V, (B, kmax)), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)
    print("[repeat] sampling walk", flush=True)
    _repeat(lambda: gdv.spec_sample_accept(drafts, k, None, V, q_tok, q_prob, lse, z, sp, sr, row_ctr, 11, pos,
                                           pos_out, acc, ne, emit, nt, st), [pos_out, acc, ne, emit, nt, st],
            "sampling walk")
    zd = torch.empty((R, V), device=dev)
    print("[repeat] dense sampling pass", flush=True)
    _repeat(lambda: gdv.spec_lm_head_sample_dense(x.hidden, wp, V, 0.9, row_ctr, 11, lse, sp, zd, workspace_buf=ws),
            [lse, sp, zd], "dense sampling pass")
    q = torch.softmax(zd * 0.8, dim=1).contiguous()
    wsd = gdv.workspace(gdv.sample_accept_dense_workspace_bytes(B), dev)
    print("[repeat] dense walk", flush=True)
    _repeat(lambda: gdv.spec_sample_accept_dense(drafts, k, None, q, zd, lse, sp, row_ctr, 11, pos, pos_out, acc, ne,
                                                 emit, nt, st, workspace_buf=wsd), [pos_out, acc, ne, emit, nt, st],
            "dense walk")


def test_delta_modes_repeat(dev):
    """DeltaNet record + fused rollback, rollback alone, VERIFY and RESCAN on the
    benchmark's workload (B=32, T=5, 32 heads), each call from a fresh copy of S_0."""
    import greedy_draft_verify_amd as gdv
    d = synth.make_delta_inputs(seed=3, device=dev)
    rec = torch.empty((d.B, d.T, d.Hd, d.dv, d.dk), dtype=torch.float32, device=dev)
    o = torch.empty((d.B, d.T, d.Hd, d.dv), dtype=torch.bfloat16, device=dev)
    L = _i32(d.L, dev)
    st = d.state.clone()

    def run(mode):
        def f():
            st.copy_(d.state)
            if mode == gdv.DELTA_ROLLBACK:
                gdv.spec_delta_verify_rollback(mode, None, None, None, None, None, 1.0, st, rec, L, None)
            elif mode == gdv.DELTA_RESCAN:
                gdv.spec_delta_verify_rollback(mode, d.q, d.k, d.v, d.a, d.b, 1.0, st, None, L, None)
            elif mode == gdv.DELTA_VERIFY:
                gdv.spec_delta_verify_rollback(mode, d.q, d.k, d.v, d.a, d.b, 1.0, st, None, None, o)
            else:
                gdv.spec_delta_verify_rollback(mode, d.q, d.k, d.v, d.a, d.b, 1.0, st, rec, L, o)
        return f

    for mode, name, outs in ((gdv.DELTA_BOTH, "record + rollback", [rec, o, st]),
                             (gdv.DELTA_ROLLBACK, "rollback", [st]),
                             (gdv.DELTA_VERIFY, "verify", [o, st]),
                             (gdv.DELTA_RESCAN, "re-scan", [st])):
        print(f"[repeat] delta {name}", flush=True)
        _repeat(run(mode), outs, f"delta {name}")
