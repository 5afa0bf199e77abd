"""The verify step captured as a HIP graph and replayed gives the eager step's bytes.

The benchmark times graph replays of spec_verify_attn -> spec_lm_head_argmax ->
spec_greedy_accept. This test captures that step for the b16k4 workload (the
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


@pytest.mark.parametrize("name", ["b16k4", "ragged"])
def test_graph_replay_matches_eager(name):
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
