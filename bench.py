"""Benchmark of one verify step on one MI355X.

A step is the whole hot path over one batch: spec_verify_attn (KV append + paged
attention, one layer) -> spec_lm_head_argmax -> spec_greedy_accept, on the
b16k4 workload (B=16 sequences, k=4 drafts, 80 rows, context U{512..4096},
32 q / 8 kv heads, head_dim 128, hidden 4096, vocabulary 151936). Inputs are
seeded synthetic tensors already resident in HBM; drafts are the target's greedy
tokens (from an untimed pass) corrupted with probability 0.3.

The timed step is a HIP graph replay of the three calls (captured once after an
eager timed loop of the same calls; the replay must reproduce the eager outputs
byte for byte). Prints one JSON line: verify rows/s (value), emitted tokens/s, the
eager per-call times, the roofline of the
dominant kernel (lm_head, weight-stream bound at 80 rows) measured with HIP events
on the launch stream, the attention roofline, and the CPU oracle timed on a bounded
sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import greedy_draft_verify_amd as gdv  # noqa: E402
from greedy_draft_verify_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)


class VerifyStep:
    """Device buffers and the three launches of one verify step (on the current
    stream, so that the same calls run eagerly or under HIP graph capture)."""

    def __init__(self, x: synth.VerifyInputs, dev, w_packed=None):
        wl = x.wl
        self.x, self.dev = x, dev
        self.B, self.R = len(x.pos), x.R
        self.q, self.k_new, self.v_new = x.q, x.k_new, x.v_new
        self.k_pool, self.v_pool = x.k_pool, x.v_pool
        self.page_table = i32(x.page_table, dev)
        self.pos, self.k = i32(x.pos, dev), i32(x.k, dev)
        self.hidden = x.hidden
        # one-time weight re-layout, outside the timed loop
        self.w_packed = gdv.spec_lm_head_pack(x.w) if w_packed is None else w_packed
        self.attn_out = torch.empty((x.R, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
        self.attn_status = torch.empty(self.B, dtype=torch.int32, device=dev)
        self.attn_ws = gdv.workspace(gdv.verify_attn_workspace_bytes(self.B, x.R, wl.Hq, wl.Hkv, wl.D,
                                                                     x.page_table.shape[1]), dev)
        self.argmax = torch.empty(x.R, dtype=torch.int32, device=dev)
        self.maxval = torch.empty(x.R, dtype=torch.float32, device=dev)
        self.lm_ws = gdv.workspace(gdv.lm_head_argmax_workspace_bytes(x.R, wl.H, wl.V), dev, zero=True)
        self.d2t = None if x.d2t is None else i32(x.d2t, dev)
        e = lambda: torch.empty(self.B, dtype=torch.int32, device=dev)
        self.pos_out, self.acc_len, self.n_emit, self.next_tok, self.acc_status = e(), e(), e(), e(), e()
        self.emit = torch.empty((self.B, wl.kmax + 1), dtype=torch.int32, device=dev)
        self.drafts = None
        # the timed step takes the lm_head and the acceptance as one call
        # (spec_lm_head_argmax_accept: the same bytes as the two calls in turn)
        self.fused = True

    def attn(self):
        gdv.spec_verify_attn(self.q, self.k_new, self.v_new, self.k_pool, self.v_pool, self.page_table,
                             self.pos, self.k, self.x.wl.kmax, self.x.scale, self.attn_out, self.attn_status,
                             workspace_buf=self.attn_ws)

    def lm_head(self):
        gdv.spec_lm_head_argmax(self.hidden, self.w_packed, self.x.wl.V, self.argmax, self.maxval,
                                workspace_buf=self.lm_ws)

    def lm_head_accept(self):
        gdv.spec_lm_head_argmax_accept(self.hidden, self.w_packed, self.x.wl.V, self.argmax, self.maxval,
                                       self.drafts, self.k, self.d2t, self.pos, self.pos_out, self.acc_len,
                                       self.n_emit, self.emit, self.next_tok, self.acc_status,
                                       workspace_buf=self.lm_ws)

    def lm_ops(self):
        """Names of the timed step's second and third calls (the third absent when fused)."""
        return ("spec_lm_head_argmax_accept", None) if self.fused else ("spec_lm_head_argmax", "spec_greedy_accept")

    def accept(self):
        gdv.spec_greedy_accept(self.argmax, self.drafts, self.k, self.d2t, self.x.wl.V, self.pos, self.pos_out,
                               self.acc_len, self.n_emit, self.emit, self.next_tok, self.acc_status)

    def outputs(self):
        """Copies of everything the step writes."""
        return [t.clone() for t in (self.attn_out, self.attn_status, self.argmax, self.maxval, self.pos_out,
                                    self.acc_len, self.n_emit, self.emit, self.next_tok, self.acc_status)]


def attn_bytes(x: synth.VerifyInputs) -> int:
    """Algorithmic bytes of one spec_verify_attn: every cached K/V byte of the attended
    positions once per (sequence, kv head), q read, output written, new K/V read and
    written once."""
    wl = x.wl
    kv = int(((x.pos.astype(np.int64) + x.k + 1) * wl.Hkv * wl.D * 2 * 2).sum())
    return kv + x.R * wl.Hq * wl.D * 2 * 2 + x.R * wl.Hkv * wl.D * 2 * 2 * 2


def lm_head_bytes(R, H, V) -> int:
    """W once + hidden once + (argmax, maxval) per row."""
    return V * H * 2 + R * H * 2 + R * 8


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of a kernel
    (calibrated FETCH_SIZE + WRITE_SIZE), or None when the summary is missing or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_key}_b16k4_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if " = " in line:
            a, b = line.split(" = ", 1)
            kv[a.strip()] = b.split()[0]
    src = os.path.join(ROOT, kv.get("source", ""))
    if not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv.get("source_sha256_16"):
        return None
    return float(kv["traffic_bytes_per_launch"])


SETTLE_S = 0.04


def settle(fn, seconds: float = SETTLE_S) -> int:
    """Untimed calls of fn, back to back, for at least `seconds`, made right before a
    timed region. After an idle spell of a few ms (a graph capture, a host-side check)
    the MI355X needs ~25 ms of load to return to its steady clocks: 20-step windows of
    the b16k4 step opened 5 steps after such a spell measure 243-253 us, the same
    windows after 100 steps 235 us. Returns the number of calls."""
    t0, n, batch = time.perf_counter(), 0, 4
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        n += batch
        batch = min(2 * batch, 64)
    return n


def time_call(f, reps: int, warmup: int = 3) -> float:
    """Mean seconds per call of f over reps back-to-back calls (HIP events on the current
    stream), after the warmup calls and the settle phase."""
    for _ in range(warmup):
        f()
    settle(f)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps / 1e3


def time_verify_step(step: VerifyStep, steps: int, warmup: int) -> dict:
    """Times one verify step: an eager loop of the three calls with HIP events on the
    launch stream around each call, then the same step captured once as a HIP graph
    and replayed (the launches' host overhead and gaps leave the step). Each timed
    region follows the warmup steps and the settle phase. Every replay must reproduce
    the eager step's bytes."""
    stream = torch.cuda.current_stream()

    def run_step(ev=None):
        if ev:
            ev[0].record(stream)
        step.attn()
        if ev:
            ev[1].record(stream)
        if step.fused:
            step.lm_head_accept()
        else:
            step.lm_head()
        if ev:
            ev[2].record(stream)
        if not step.fused:
            step.accept()
        if ev:
            ev[3].record(stream)

    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    assert (step.attn_status.cpu() == 0).all() and (step.acc_status.cpu() == 0).all()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle_eager = settle(run_step)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        run_step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / steps
    eager_out = step.outputs()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run_step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run_step()
    for _ in range(warmup):
        graph.replay()
    settle_graph = settle(graph.replay)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop) / steps
    for a, b in zip(eager_out, step.outputs()):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "graph replay differs from the eager step"
    del graph
    return {"graph_ms": graph_ms, "eager_ms": eager_ms, "settle_steps": [settle_eager, settle_graph],
            "attn_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
            "lm_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
            "acc_ms": float(np.mean([e[2].elapsed_time(e[3]) for e in evs])),
            "median_us": {name: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3
                          for i, name in enumerate(("spec_verify_attn",) + step.lm_ops()) if name}}


def step_report(step: VerifyStep, t: dict) -> dict:
    """Rates and rooflines of a timed verify step."""
    x, wl = step.x, step.x.wl
    acc_len = step.acc_len.cpu().numpy()
    emitted = int((acc_len + 1).sum())
    lm_b = lm_head_bytes(x.R, wl.H, wl.V)
    at_b = attn_bytes(x)
    lm_gbs = lm_b / (t["lm_ms"] / 1e3) / 1e9
    at_gbs = at_b / (t["attn_ms"] / 1e3) / 1e9
    lm_tflops = 2.0 * x.R * wl.H * wl.V / (t["lm_ms"] / 1e3) / 1e12
    return {"rows": x.R, "step_us": t["graph_ms"] * 1e3, "eager_step_us": t["eager_ms"] * 1e3,
            "lm_us": (t["lm_ms"] + (0.0 if step.fused else t["acc_ms"])) * 1e3,
            "rows_per_s": x.R / (t["graph_ms"] / 1e3), "emitted_tokens_per_s": emitted / (t["graph_ms"] / 1e3),
            "emitted_per_step": emitted,
            "accept_len_hist": np.bincount(acc_len, minlength=wl.kmax + 1).tolist(),
            "kernel_us": {name: v for name, v in zip(("spec_verify_attn",) + step.lm_ops(),
                                                     (t["attn_ms"] * 1e3, t["lm_ms"] * 1e3, t["acc_ms"] * 1e3))
                          if name},
            "kernel_us_median": t["median_us"],
            "attn": {"bound": "hbm", "algorithmic_bytes": at_b, "achieved": at_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": at_gbs / HBM_PEAK_GBS},
            "lm_head": {"bound": "hbm" if x.R < 312 else "mfma", "algorithmic_bytes": lm_b, "GB/s": lm_gbs,
                        "hbm_frac": lm_gbs / HBM_PEAK_GBS, "TFLOP/s": lm_tflops,
                        "mfma_frac": lm_tflops / BF16_PEAK_TFLOPS}}


def config_leg(name: str, dev, steps: int, warmup: int, seed: int = 0) -> dict:
    """The verify step (attention + lm_head + accept) on another workload, timed as the
    headline step is. Drafts: the greedy tokens of an untimed lm_head pass, corrupted
    per position (the parity tests use the oracle's greedy tokens; the two agree on
    every row whose top-2 gap exceeds 5e-2)."""
    x = synth.make_verify_inputs(name, seed=seed, device=dev)
    wl = x.wl
    step = VerifyStep(x, dev)
    x.w = None
    torch.cuda.empty_cache()
    step.lm_head()
    torch.cuda.synchronize()
    g0 = step.argmax.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    step.drafts = i32(synth.make_drafts(wl, x.k, [g0[off[s]:off[s] + x.k[s]] for s in range(len(x.pos))],
                                        seed=seed, d2t=x.d2t), dev)
    rep = step_report(step, time_verify_step(step, steps, warmup))
    ctx = f"U{{{wl.ctx_lo}..{wl.ctx_hi}}}" if wl.ctx_lo != wl.ctx_hi else str(wl.ctx_lo)
    ks = f"k={wl.k}" if wl.k is not None else f"k_s ~ U{{{wl.k_lo}..{wl.k_hi}}}"
    rep = {"workload": f"{name}: B={len(x.pos)}, {ks}, context {ctx}, {wl.Hq}q/{wl.Hkv}kv heads, head_dim {wl.D}, "
                       f"hidden {wl.H}, vocab {wl.V}" + (f", d2t {len(x.d2t)} entries" if x.d2t is not None else ""),
           "kv_split_tokens": gdv.attn_split_tokens(x.page_table.shape[1]), **rep}
    log(f"[bench] {name}: step {rep['step_us']:.1f} us ({rep['rows_per_s']:.0f} rows/s, "
        f"{rep['emitted_tokens_per_s']:.0f} tokens/s): attn {rep['kernel_us']['spec_verify_attn']:.1f} us "
        f"({100 * rep['attn']['frac']:.0f}% HBM), lm_head+accept {rep['lm_us']:.1f} us "
        f"({100 * rep['lm_head']['hbm_frac']:.0f}% HBM, {100 * rep['lm_head']['mfma_frac']:.0f}% MFMA)")
    del step, x
    torch.cuda.empty_cache()
    return rep


def delta_leg(dev, reps: int):
    """Gated DeltaNet verify with per-token record and fused rollback (mode BOTH) on the
    hybrid workload: B=32, T=5, 32 heads, 128x128 fp32 state. Algorithmic bytes: S_0
    read, every S_t recorded, q/k/v/a/b read, o written, S_L written for L > 0. Beside
    it the input-stash pair: VERIFY (outputs only) and RESCAN (the committed prefix
    re-run from the retained S_0)."""
    d = synth.make_delta_inputs(seed=0, device=dev)
    st_bytes = d.dv * d.dk * 4
    rec = torch.empty((d.B, d.T, d.Hd, d.dv, d.dk), dtype=torch.float32, device=dev)
    o = torch.empty((d.B, d.T, d.Hd, d.dv), dtype=torch.bfloat16, device=dev)
    L = i32(d.L, dev)
    state = d.state.clone()
    f = lambda: gdv.spec_delta_verify_rollback(gdv.DELTA_BOTH, d.q, d.k, d.v, d.a, d.b, 1.0, state, rec, L, o)
    sec = time_call(f, reps)
    n_sh = d.B * d.Hd
    byts = (n_sh * st_bytes * (1 + d.T) + d.B * d.T * d.Hd * (2 * d.dk + d.dv) * 2 + d.B * d.T * d.Hd * 8
            + d.B * d.T * d.Hd * d.dv * 2 + int((d.L > 0).sum()) * d.Hd * st_bytes)
    gbs = byts / sec / 1e9
    restore = lambda: gdv.spec_delta_verify_rollback(gdv.DELTA_ROLLBACK, None, None, None, None, None, 1.0, state,
                                                     rec, L, None)
    sec_r = time_call(restore, reps)
    byts_r = 2 * int((d.L > 0).sum()) * d.Hd * st_bytes
    # input-stash alternative: verify writes outputs only; a partial accept re-runs the
    # committed prefix from the retained S_0 (re-reads S_0, writes S_L)
    s0 = d.state.clone()
    ver = lambda: gdv.spec_delta_verify_rollback(gdv.DELTA_VERIFY, d.q, d.k, d.v, d.a, d.b, 1.0, s0, None, None, o)
    sec_v = time_call(ver, reps)
    byts_v = (n_sh * st_bytes + d.B * d.T * d.Hd * (2 * d.dk + d.dv) * 2 + d.B * d.T * d.Hd * 8
              + d.B * d.T * d.Hd * d.dv * 2)
    s5 = d.state.clone()
    resc = lambda: gdv.spec_delta_verify_rollback(gdv.DELTA_RESCAN, d.q, d.k, d.v, d.a, d.b, 1.0, s5, None, L)
    sec_s = time_call(resc, reps)
    n_l = int((d.L > 0).sum())
    byts_s = (2 * n_l * d.Hd * st_bytes + int(d.L.sum()) * d.Hd * ((2 * d.dk + d.dv) * 2 + 8))
    return {"workload": f"B={d.B} T={d.T} heads={d.Hd} state {d.dv}x{d.dk} fp32, L ~ U{{0..{d.T}}}",
            "verify_record_rollback_us": sec * 1e6, "algorithmic_bytes": byts, "achieved": gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "bound": "hbm",
            "rollback_only_us": sec_r * 1e6, "rollback_only_bytes": byts_r,
            "rollback_only_frac": byts_r / sec_r / 1e9 / HBM_PEAK_GBS,
            "input_stash": {"verify_us": sec_v * 1e6, "verify_bytes": byts_v,
                            "verify_frac": byts_v / sec_v / 1e9 / HBM_PEAK_GBS,
                            "rescan_us": sec_s * 1e6, "rescan_bytes": byts_s,
                            "rescan_frac": byts_s / sec_s / 1e9 / HBM_PEAK_GBS,
                            "total_us": (sec_v + sec_s) * 1e6},
            # one round at this workload's L mix: record every state and restore by the
            # fused copy, or keep the inputs and re-run the committed prefix
            "per_round_us": {"record": sec * 1e6, "stash": (sec_v + sec_s) * 1e6}}


def tree_leg(dev, w_packed, reps: int, seed: int = 0):
    """Tree drafts on the b16k4 shapes (DSSD fast.py _tree_cycle): 16 sequences with a
    16-node trie each (a spine of 8 head drafts, then side branches), 256 rows. One
    tree step = spec_verify_attn_tree -> spec_lm_head_argmax (the workload's W) ->
    spec_tree_accept -> spec_kv_compact, each timed with HIP events on the launch
    stream; beside it the chain attention over the same 256 rows (k = 15) for the cost
    of the ancestor masks."""
    x = synth.make_verify_inputs("b16tree", seed=seed, device=dev, with_lm_head=False)
    wl = x.wl
    B, R, kmax = len(x.pos), x.R, wl.kmax
    hidden = synth.normal_bf16((R, wl.H), 1.0, seed, wl.name, "hidden", dev)
    parent_np = synth.make_parents(x.k, seed, wl.name, "trie")
    parent = i32(parent_np, dev)
    pt, pos, k = i32(x.page_table, dev), i32(x.pos, dev), i32(x.k, dev)
    out = torch.empty((R, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    ws_t = gdv.workspace(gdv.verify_attn_tree_workspace_bytes(B, R, wl.Hq, wl.Hkv, wl.D, x.page_table.shape[1],
                                                              kmax), dev)
    ws_c = gdv.workspace(gdv.verify_attn_workspace_bytes(B, R, wl.Hq, wl.Hkv, wl.D, x.page_table.shape[1]), dev)
    attn_t = lambda: gdv.spec_verify_attn_tree(x.q, x.k_new, x.v_new, x.k_pool, x.v_pool, pt, pos, k, parent,
                                               x.scale, out, st, workspace_buf=ws_t)
    attn_c = lambda: gdv.spec_verify_attn(x.q, x.k_new, x.v_new, x.k_pool, x.v_pool, pt, pos, k, kmax, x.scale,
                                          out, st, workspace_buf=ws_c)
    am = torch.empty(R, dtype=torch.int32, device=dev)
    lm_ws = gdv.workspace(gdv.lm_head_argmax_workspace_bytes(R, wl.H, wl.V), dev, zero=True)
    lm = lambda: gdv.spec_lm_head_argmax(hidden, w_packed, wl.V, am, None, workspace_buf=lm_ws)
    lm()
    attn_t()
    torch.cuda.synchronize()
    assert (st.cpu() == 0).all()
    g0 = am.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    drafts = i32(synth.make_tree_drafts(wl, x.k, parent_np, [g0[off[s]:off[s + 1]] for s in range(B)], seed), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, ast = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)
    path = torch.empty((B, kmax), dtype=torch.int32, device=dev)
    cst = torch.zeros(B, dtype=torch.int32, device=dev)
    accept = lambda: gdv.spec_tree_accept(am, drafts, k, parent, None, wl.V, pos, pos_out, acc, ne, emit, nt, path,
                                          ast)
    compact = lambda: gdv.spec_kv_compact(x.k_pool, x.v_pool, pt, pos, path, acc, cst.zero_())
    stream = torch.cuda.current_stream()
    fns = [attn_t, lm, accept, compact]
    for _ in range(3):
        for f in fns:
            f()
    torch.cuda.synchronize()
    assert (ast.cpu() == 0).all() and (cst.cpu() == 0).all()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    settle(lambda: [f() for f in fns])
    for ev in evs:
        ev[0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = [float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in evs])) * 1e3 for i in range(len(fns))]
    # the chain attention over the same rows, timed in the same place (after an lm_head
    # pass has streamed W through the caches)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for ev in evc:
        lm()
        ev[0].record(stream)
        attn_c()
        ev[1].record(stream)
    torch.cuda.synchronize()
    chain_us = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in evc])) * 1e3
    acc_np = acc.cpu().numpy()
    at_b = attn_bytes(x)
    cmp_b = int(acc_np.sum()) * wl.Hkv * wl.D * 2 * 2 * 2
    step_us = sum(us)
    return {"workload": f"b16tree: B={B}, 16-node trie per sequence (spine 8 + branches), R={R}, context "
                        f"U{{{wl.ctx_lo}..{wl.ctx_hi}}}, {wl.Hq}q/{wl.Hkv}kv, head_dim {wl.D}, vocab {wl.V}",
            "step_us": step_us, "rows_per_s": R / (step_us / 1e6),
            "emitted_tokens_per_s": float((acc_np + 1).sum()) / (step_us / 1e6),
            "accept_len_hist": np.bincount(acc_np, minlength=kmax + 1).tolist(),
            "kernel_us": {"spec_verify_attn_tree": us[0], "spec_lm_head_argmax": us[1], "spec_tree_accept": us[2],
                          "spec_kv_compact": us[3]},
            "attn_tree": {"bound": "hbm", "algorithmic_bytes": at_b, "achieved": at_b / us[0] / 1e3,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": at_b / us[0] / 1e3 / HBM_PEAK_GBS},
            "attn_chain_same_rows_us": chain_us,
            "kv_compact_bytes": cmp_b}


def sampling_leg(step: "VerifyStep", dev, reps: int, temperature: float = 0.1):
    """Speculative-sampling verify on the benchmark's inputs (DSSD fast.py
    _sample_verify): spec_verify_attn -> spec_lm_head_sample (softmax statistics and
    the two Gumbel-max draws fused into the lm_head pass) -> spec_sample_accept, with
    point-mass draft distributions at the step's drafts. The synthetic logits have unit
    variance over 151936 entries, nearly flat at temperature 1 (a greedy draft is kept
    with probability ~1e-4 there), so the leg runs at temperature 0.1. Each call timed
    with HIP events on the launch stream."""
    x = step.x
    wl = x.wl
    B, R, kmax = step.B, step.R, wl.kmax
    drafts = step.drafts.cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    q_tok = np.full((R, 1), -1, np.int32)
    for s in range(B):
        q_tok[off[s]:off[s] + x.k[s], 0] = drafts[s, :x.k[s]] if x.d2t is None else x.d2t[drafts[s, :x.k[s]]]
    q_prob = torch.from_numpy((q_tok >= 0).astype(np.float32)).to(dev)
    q_tok_d = i32(q_tok, dev)
    row_ctr = i32(np.stack([np.concatenate([x.pos[s] + np.arange(x.k[s] + 1) for s in range(B)]),
                            np.repeat(np.arange(B), x.k + 1)], 1), dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    z_supp = torch.empty((R, 1), dtype=torch.float32, device=dev)
    sp = torch.empty(R, dtype=torch.int32, device=dev)
    sr = torch.empty(R, dtype=torch.int32, device=dev)
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, wl.H, wl.V), dev, zero=True)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)
    seed = 0x5EED
    lm = lambda: gdv.spec_lm_head_sample(x.hidden, step.w_packed, wl.V, temperature, q_tok_d, q_prob, row_ctr, seed,
                                         lse, z_supp, sp, sr, workspace_buf=ws)
    accept = lambda: gdv.spec_sample_accept(step.drafts, step.k, step.d2t, wl.V, q_tok_d, q_prob, lse, z_supp, sp,
                                            sr, row_ctr, seed, step.pos, pos_out, acc, ne, emit, nt, st)
    fns = [step.attn, lm, accept]
    stream = torch.cuda.current_stream()
    for _ in range(3):
        for f in fns:
            f()
    torch.cuda.synchronize()
    assert (st.cpu() == 0).all()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    settle(lambda: [f() for f in fns])
    for ev in evs:
        ev[0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = [float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in evs])) * 1e3 for i in range(len(fns))]
    acc_np = acc.cpu().numpy()
    step_us = sum(us)
    lm_b = lm_head_bytes(R, wl.H, wl.V)
    return {"workload": f"{wl.name} inputs, temperature {temperature}, point-mass drafts",
            "step_us": step_us, "rows_per_s": R / (step_us / 1e6),
            "emitted_tokens_per_s": float((acc_np + 1).sum()) / (step_us / 1e6),
            "accept_len_hist": np.bincount(acc_np, minlength=kmax + 1).tolist(),
            "kernel_us": {"spec_verify_attn": us[0], "spec_lm_head_sample": us[1], "spec_sample_accept": us[2]},
            "lm_head_sample": {"bound": "hbm", "algorithmic_bytes": lm_b, "achieved": lm_b / us[1] / 1e3,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": lm_b / us[1] / 1e3 / HBM_PEAK_GBS}}


def sampling_dense_leg(step: "VerifyStep", dev, reps: int, temperature: float = 0.1):
    """Speculative sampling with dense draft distributions (DSSD fast.py _sample_verify
    with the draft head's whole q): spec_verify_attn -> spec_lm_head_sample_dense (the
    pass also writes z = logit / T of every entry, R x V fp32) -> spec_sample_accept_dense
    (the walk, then the residual of each rejected row drawn over the whole vocabulary).
    Setup, untimed: z from one pass, q = softmax(0.8 z + N(0, 1)) per row (a draft
    distribution near the target), each draft drawn from its row's q."""
    x = step.x
    wl = x.wl
    B, R, kmax, V = step.B, step.R, wl.kmax, wl.V
    row_ctr = i32(np.stack([np.concatenate([x.pos[s] + np.arange(x.k[s] + 1) for s in range(B)]),
                            np.repeat(np.arange(B), x.k + 1)], 1), dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    sp = torch.empty(R, dtype=torch.int32, device=dev)
    z = torch.empty((R, V), dtype=torch.float32, device=dev)
    ws = gdv.workspace(gdv.lm_head_sample_workspace_bytes(R, wl.H, V), dev, zero=True)
    seed = 0xD5EED
    lm = lambda: gdv.spec_lm_head_sample_dense(x.hidden, step.w_packed, V, temperature, row_ctr, seed, lse, sp, z,
                                               workspace_buf=ws)
    lm()
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    q = torch.softmax(0.8 * z + torch.randn((R, V), generator=gen, device=dev), dim=1).contiguous()
    draws = torch.multinomial(q, 1, generator=gen).to(torch.int32).view(-1).cpu().numpy()
    off = np.concatenate([[0], np.cumsum(x.k + 1)])
    drafts_np = np.zeros((B, kmax), np.int32)
    for s in range(B):
        drafts_np[s, :x.k[s]] = draws[off[s]:off[s] + x.k[s]]
    drafts = i32(drafts_np, dev)
    wsd = gdv.workspace(gdv.sample_accept_dense_workspace_bytes(B), dev)
    e = lambda: torch.empty(B, dtype=torch.int32, device=dev)
    pos_out, acc, ne, nt, st = e(), e(), e(), e(), e()
    emit = torch.empty((B, kmax + 1), dtype=torch.int32, device=dev)
    accept = lambda: gdv.spec_sample_accept_dense(drafts, step.k, None, q, z, lse, sp, row_ctr, seed, step.pos,
                                                  pos_out, acc, ne, emit, nt, st, workspace_buf=wsd)
    fns = [step.attn, lm, accept]
    stream = torch.cuda.current_stream()
    for _ in range(3):
        for f in fns:
            f()
    torch.cuda.synchronize()
    assert (st.cpu() == 0).all()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    settle(lambda: [f() for f in fns])
    for ev in evs:
        ev[0].record(stream)
        for i, f in enumerate(fns):
            f()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    us = [float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in evs])) * 1e3 for i in range(len(fns))]
    acc_np = acc.cpu().numpy()
    step_us = sum(us)
    lm_b = lm_head_bytes(R, wl.H, V) + R * V * 4          # + z written
    rejected = int((acc_np < x.k).sum())
    acc_b = rejected * V * 8 + R * 12                    # rejected rows' z and q, per-draft lookups
    return {"workload": f"{wl.name} inputs, temperature {temperature}, dense q = softmax(0.8 z + N(0,1))",
            "step_us": step_us, "rows_per_s": R / (step_us / 1e6),
            "emitted_tokens_per_s": float((acc_np + 1).sum()) / (step_us / 1e6),
            "accept_len_hist": np.bincount(acc_np, minlength=kmax + 1).tolist(),
            "rejected_sequences": rejected,
            "kernel_us": {"spec_verify_attn": us[0], "spec_lm_head_sample_dense": us[1],
                          "spec_sample_accept_dense": us[2]},
            "lm_head_sample_dense": {"bound": "hbm", "algorithmic_bytes": lm_b, "achieved": lm_b / us[1] / 1e3,
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": lm_b / us[1] / 1e3 / HBM_PEAK_GBS},
            "accept_dense_bytes": acc_b}


def kpolicy_leg(step: "VerifyStep", dev, reps: int, seed: int = 0):
    """The verify cost against rows that drives the adaptive draft depth (span-02
    KPolicy): the b16k4 step (attention + lm_head + accept) at B = 16 with k = 0..7
    drafts per sequence (16..128 rows), each call timed with events in the step's own
    order; then the library policy's choice of k for a few acceptance rates and draft
    costs."""
    base = step.x.wl
    table = []
    for k in range(8):
        wl = synth.VerifyWorkload(f"b16k{k}", B=16, k=k, k_lo=k, k_hi=k, ctx_lo=base.ctx_lo, ctx_hi=base.ctx_hi,
                                  Hq=base.Hq, Hkv=base.Hkv, D=base.D, H=base.H, V=base.V, max_pages=base.max_pages,
                                  w_std=base.w_std)
        x = synth.make_verify_inputs(wl, seed=seed, device=dev, with_lm_head=False)
        x.hidden = synth.normal_bf16((x.R, wl.H), 1.0, seed, "b16k4", "extra", dev)
        st = VerifyStep(x, dev, w_packed=step.w_packed)
        st.drafts = i32(np.zeros((16, max(k, 1)), np.int32)[:, :k] if k else np.zeros((16, 0), np.int32), dev)
        fns = [st.attn, st.lm_head, st.accept]
        stream = torch.cuda.current_stream()
        for _ in range(3):
            for f in fns:
                f()
        settle(lambda: [f() for f in fns])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for f in fns:
                f()
        e1.record(stream)
        torch.cuda.synchronize()
        table.append((x.R, e0.elapsed_time(e1) / reps * 1e3))
        del st, x
        torch.cuda.empty_cache()
    choices = []
    for p in (0.3, 0.5, 0.7, 0.9):
        for draft_us in (0.0, 15.0, 50.0):
            pol = gdv.KPolicy(kmin=0, kmax=7, prior_p=p, prior_n=1e12, draft_us=draft_us, table=table)
            k = pol.choose(16)
            choices.append({"accept_p": p, "draft_us": draft_us, "k": k,
                            "us_per_token": (pol.verify_cost(16 * (k + 1)) + k * draft_us) / pol.expected_tokens(k)
                            / 16})
    return {"workload": "b16k4 shapes at B=16, k = 0..7", "verify_us_by_rows": table, "choices": choices}


def lm_head_sweep(x: synth.VerifyInputs, w_packed, dev, reps: int):
    """spec_lm_head_argmax alone at growing row counts with the workload's W: where the
    weight stream stops bounding it and the MFMA work starts to."""
    wl = x.wl
    out = []
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    for R in (80, 160, 288, 311, 512, 1024):
        h = torch.randn((R, wl.H), generator=g, device=dev).to(torch.bfloat16)
        am = torch.empty(R, dtype=torch.int32, device=dev)
        ws = gdv.workspace(gdv.lm_head_argmax_workspace_bytes(R, wl.H, wl.V), dev, zero=True)
        sec = time_call(lambda: gdv.spec_lm_head_argmax(h, w_packed, wl.V, am, None, workspace_buf=ws), reps)
        tf = 2.0 * R * wl.H * wl.V / sec / 1e12
        gbs = lm_head_bytes(R, wl.H, wl.V) / sec / 1e9
        out.append({"rows": R, "us": sec * 1e6, "GB/s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "TFLOP/s": tf,
                    "mfma_frac": tf / BF16_PEAK_TFLOPS})
    return out


def cpu_baseline(x_host: synth.VerifyInputs, n_seq: int, min_seconds: float = 10.0):
    """The CPU oracle on the first n_seq sequences of the workload (same inputs)."""
    import oracle
    wl = x_host.wl
    bits = synth.bf16_bits
    seqs = list(range(n_seq))
    off_all = np.concatenate([[0], np.cumsum(x_host.k + 1)]).astype(np.int64)
    rows = np.concatenate([np.arange(off_all[s], off_all[s + 1]) for s in seqs])
    R = len(rows)
    pos, k, pt = x_host.pos[seqs], x_host.k[seqs], x_host.page_table[seqs]
    kp, vp = bits(x_host.k_pool).copy(), bits(x_host.v_pool).copy()
    qb, knb, vnb = bits(x_host.q)[rows], bits(x_host.k_new)[rows], bits(x_host.v_new)[rows]
    hb, wb = bits(x_host.hidden)[rows], bits(x_host.w)
    oracle.lib()
    # the whole oracle step, repeated until at least min_seconds of CPU work (the
    # mean per repetition is reported)
    t_attn = t_lm = t_acc = 0.0
    reps = 0
    while reps == 0 or t_attn + t_lm + t_acc < min_seconds:
        kpr, vpr = kp.copy(), vp.copy()
        t0 = time.perf_counter()
        off, st = oracle.validate(pt, pt.shape[1], x_host.n_pages, pos, k, wl.kmax, n_seq, R)
        oracle.append_kv(knb, vnb, kpr, vpr, pt, pt.shape[1], pos, k, off, st, n_seq, wl.Hkv, wl.D)
        oracle.verify_attn(qb, kpr, vpr, pt, pt.shape[1], pos, k, off, st, n_seq, R, wl.Hq, wl.Hkv, wl.D,
                           x_host.scale)
        t1 = time.perf_counter()
        g, _, _, _ = oracle.lm_head_argmax(hb, wb, R, wl.H, wl.V)
        t2 = time.perf_counter()
        if reps == 0:
            true_next = [g[off[s]:off[s] + k[s]] for s in range(n_seq)]
            drafts = synth.make_drafts(wl, k, true_next, seed=0, d2t=x_host.d2t)
        t3 = time.perf_counter()
        oracle.greedy_accept(g, drafts, wl.kmax, k, x_host.d2t, 0 if x_host.d2t is None else len(x_host.d2t),
                             wl.V, n_seq, R, pos)
        t4 = time.perf_counter()
        t_attn, t_lm, t_acc, reps = t_attn + (t1 - t0), t_lm + (t2 - t1), t_acc + (t4 - t3), reps + 1
    secs = (t_attn + t_lm + t_acc) / reps
    # threads the step actually ran on: the oracle's OpenMP pool and numpy's BLAS pool
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([int(p_.get("num_threads", 1)) for p_ in threadpool_info()] or [1])
    # the same step once more on one core (both pools limited to one thread)
    with threadpool_limits(limits=1):
        kpr, vpr = kp.copy(), vp.copy()
        t0 = time.perf_counter()
        off, st = oracle.validate(pt, pt.shape[1], x_host.n_pages, pos, k, wl.kmax, n_seq, R)
        oracle.append_kv(knb, vnb, kpr, vpr, pt, pt.shape[1], pos, k, off, st, n_seq, wl.Hkv, wl.D)
        oracle.verify_attn(qb, kpr, vpr, pt, pt.shape[1], pos, k, off, st, n_seq, R, wl.Hq, wl.Hkv, wl.D,
                           x_host.scale)
        g, _, _, _ = oracle.lm_head_argmax(hb, wb, R, wl.H, wl.V)
        oracle.greedy_accept(g, drafts, wl.kmax, k, x_host.d2t, 0 if x_host.d2t is None else len(x_host.d2t),
                             wl.V, n_seq, R, pos)
        secs_1 = time.perf_counter() - t0
    model = "unknown CPU"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    g_all, t1_all, t2_all = oracle.lm_head_argmax(hb, wb, R, wl.H, wl.V)[:3]
    return dict(value=R / secs, unit="rows/s", cores=cores, kind="oracle",
                sample=f"first {n_seq} of {len(x_host.pos)} sequences ({R} rows), the whole oracle step "
                       f"repeated {reps} times ({t_attn + t_lm + t_acc:.1f} s); per repetition: fp64 "
                       f"attention+append {t_attn / reps:.3f}s, lm_head+argmax {t_lm / reps:.3f}s, accept "
                       f"{t_acc / reps:.5f}s; host: {model}, os.cpu_count() = {os.cpu_count()}",
                single_core_value=R / secs_1, single_core_seconds=secs_1,
                seconds=secs, greedy=(rows, g_all, t1_all - t2_all))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b16k4", choices=["b16k4", "ragged", "long", "tiny"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-seqs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every leg reported beside the step")
    ap.add_argument("--extras", default="configs,sweep,delta,tree,sampling,adaptive",
                    help="comma list of the legs reported beside the step: configs (the verify step on the "
                         "tiny, ragged and long workloads), sweep (lm_head rows), delta (DeltaNet), tree, "
                         "sampling, adaptive (verify cost by rows + draft-depth policy)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed loop, copy this many MiB 3 times (a plain copy kernel of known "
                         "size, used to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verify step runs on a single MI355X here "
              "(sharding is described in the design notes, not run)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    x = synth.make_verify_inputs(args.workload, seed=args.seed, device=dev)
    wl = x.wl
    log(f"[bench] {wl.name}: B={len(x.pos)} R={x.R} pos {x.pos.min()}..{x.pos.max()} pool {x.n_pages} pages, "
        f"inputs drawn in {time.perf_counter() - t_gen:.1f}s")
    off = np.concatenate([[0], np.cumsum(x.k + 1)])

    # The CPU baseline runs first, on host copies (before any append touches the
    # pool): the oracle's step on a bounded sample, whose greedy tokens also give the
    # drafts of the timed step when the sample covers every sequence.
    cpu, oracle_greedy = None, None
    if not args.no_cpu_baseline:
        x_host = synth.VerifyInputs(wl, x.pos, x.k, x.R, x.page_table, x.n_pages, x.q.cpu(), x.k_new.cpu(),
                                    x.v_new.cpu(), x.k_pool.cpu(), x.v_pool.cpu(), x.hidden.cpu(), x.w.cpu(), x.d2t)
        n_seq = min(args.cpu_sample_seqs, len(x.pos))
        log(f"[bench] cpu baseline: oracle on {n_seq} sequences ...")
        cpu = cpu_baseline(x_host, n_seq)
        log(f"[bench] cpu baseline {cpu['value']:.3f} rows/s ({cpu['sample']})")
        cpu.pop("seconds")
        rows_o, g_o, gap_o = cpu.pop("greedy")
        if len(rows_o) == x.R:
            oracle_greedy = (g_o, gap_o)
        del x_host

    step = VerifyStep(x, dev)
    x.w = None                      # the packed copy is the one the step reads
    torch.cuda.empty_cache()
    # an untimed lm_head pass: the GPU's greedy tokens, compared with the oracle's
    step.lm_head()
    torch.cuda.synchronize()
    g_gpu = step.argmax.cpu().numpy()
    drafts_note = {}
    if oracle_greedy is not None:
        g_src = oracle_greedy[0]
        diff = g_gpu != g_src
        drafts_note = {"drafts_from": "oracle greedy tokens (fp64), corrupted per position",
                       "gpu_argmax_rows_differing_from_oracle": int(diff.sum()),
                       "of_which_oracle_gap_le_5e-2": int((diff & (oracle_greedy[1] <= 5e-2)).sum())}
    else:
        g_src = g_gpu
        drafts_note = {"drafts_from": "GPU greedy tokens of an untimed lm_head pass (no CPU baseline run), "
                                      "corrupted per position"}
    true_next = [g_src[off[s]:off[s] + x.k[s]] for s in range(len(x.pos))]
    step.drafts = i32(synth.make_drafts(wl, x.k, true_next, seed=args.seed, d2t=x.d2t), dev)

    t = time_verify_step(step, args.steps, args.warmup)
    rep = step_report(step, t)
    lm_call = step.lm_ops()[0]
    ms_step = t["graph_ms"]
    lm, at = rep["lm_head"], rep["attn"]
    log(f"[bench] step {ms_step * 1e3:.1f} us (graph replay; eager {t['eager_ms'] * 1e3:.1f} us): attn "
        f"{t['attn_ms'] * 1e3:.1f} us ({at['achieved']:.0f} GB/s), lm_head+accept {rep['lm_us']:.1f} us "
        f"({lm['GB/s']:.0f} GB/s, {lm['TFLOP/s']:.1f} TFLOP/s); "
        f"accept-length histogram {rep['accept_len_hist']}; {drafts_note}")

    extras = {}
    legs = set() if args.no_extras else {e.strip() for e in args.extras.split(",") if e.strip()}
    unknown = legs - {"configs", "sweep", "delta", "tree", "sampling", "adaptive"}
    if unknown:
        raise SystemExit(f"bench.py: unknown --extras legs {sorted(unknown)}")
    if legs:
        if "sweep" in legs:
            extras["lm_head_row_sweep"] = lm_head_sweep(x, step.w_packed, dev, reps=10)
        if "tree" in legs and wl.H == 4096 and wl.V == 151936:
            extras["tree_verify"] = tree_leg(dev, step.w_packed, reps=20, seed=args.seed)
        if "sampling" in legs:
            extras["sampling_verify"] = sampling_leg(step, dev, reps=20)
            extras["sampling_dense_verify"] = sampling_dense_leg(step, dev, reps=20)
        if "adaptive" in legs and wl.name == "b16k4":
            extras["adaptive_k"] = kpolicy_leg(step, dev, reps=10, seed=args.seed)
        if "configs" in legs or "delta" in legs:
            # the other workloads of the verify step, each timed like the headline one
            # (the headline step's buffers are released first)
            del step
            torch.cuda.empty_cache()
            configs = {}
            if "configs" in legs:
                for name in ("tiny", "ragged", "long"):
                    if name != wl.name:
                        configs[name] = config_leg(name, dev, steps=max(10, args.steps // 5), warmup=args.warmup,
                                                   seed=args.seed)
            if "delta" in legs:
                configs["delta"] = delta_leg(dev, reps=20)
                dl = configs["delta"]
                ist = dl["input_stash"]
                log(f"[bench] delta verify+record+rollback {dl['verify_record_rollback_us']:.1f} us "
                    f"({dl['achieved']:.0f} GB/s, {100 * dl['frac']:.0f}% of HBM peak); rollback alone "
                    f"{dl['rollback_only_us']:.1f} us; input stash: verify {ist['verify_us']:.1f} us + re-scan "
                    f"{ist['rescan_us']:.1f} us (record+rollback vs stash per round at this L mix: "
                    f"{dl['per_round_us']['record']:.1f} vs {dl['per_round_us']['stash']:.1f} us)")
            extras["configs"] = configs
        if "lm_head_row_sweep" in extras:
            sw = ", ".join(f"R={e['rows']}: {e['us']:.0f} us {e['TFLOP/s']:.0f} TF/s" for e in extras["lm_head_row_sweep"])
            log(f"[bench] lm_head sweep: {sw}")
        if "adaptive_k" in extras:
            ak = extras["adaptive_k"]
            tbl = ", ".join(f"{r}: {t_:.0f}" for r, t_ in ak["verify_us_by_rows"])
            ch = ", ".join(f"p={c['accept_p']}/d={c['draft_us']:.0f}->k={c['k']}" for c in ak["choices"])
            log(f"[bench] verify us by rows (B=16): {tbl}; policy: {ch}")
        sv_ = extras.get("sampling_verify")
        if sv_:
            log(f"[bench] sampling step {sv_['step_us']:.1f} us ({sv_['rows_per_s']:.0f} rows/s, "
                f"{sv_['emitted_tokens_per_s']:.0f} tokens/s): lm_head+sample {sv_['kernel_us']['spec_lm_head_sample']:.1f} us "
                f"({100 * sv_['lm_head_sample']['frac']:.0f}% HBM), accept {sv_['kernel_us']['spec_sample_accept']:.1f} us; "
                f"accept lengths {sv_['accept_len_hist']}")
        sd = extras.get("sampling_dense_verify")
        if sd:
            log(f"[bench] dense sampling step {sd['step_us']:.1f} us ({sd['rows_per_s']:.0f} rows/s, "
                f"{sd['emitted_tokens_per_s']:.0f} tokens/s): lm_head+sample+z "
                f"{sd['kernel_us']['spec_lm_head_sample_dense']:.1f} us "
                f"({100 * sd['lm_head_sample_dense']['frac']:.0f}% HBM), accept+residual "
                f"{sd['kernel_us']['spec_sample_accept_dense']:.1f} us ({sd['rejected_sequences']} residual draws); "
                f"accept lengths {sd['accept_len_hist']}")
        if "tree_verify" in extras:
            tv = extras["tree_verify"]
            ku = tv["kernel_us"]
            log(f"[bench] tree step {tv['step_us']:.1f} us ({tv['rows_per_s']:.0f} rows/s, "
                f"{tv['emitted_tokens_per_s']:.0f} tokens/s): attn {ku['spec_verify_attn_tree']:.1f} us "
                f"({100 * tv['attn_tree']['frac']:.0f}% HBM; chain over the same rows "
                f"{tv['attn_chain_same_rows_us']:.1f} us), lm_head {ku['spec_lm_head_argmax']:.1f} us, accept "
                f"{ku['spec_tree_accept']:.1f} us, compact {ku['spec_kv_compact']:.1f} us; accept lengths "
                f"{tv['accept_len_hist']}")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    lm_frac = lm["hbm_frac"] if lm["bound"] == "hbm" else lm["mfma_frac"]
    result = {
        "metric": "verify rows/s (B=16, k=4; emitted tokens/s and roofline fractions alongside)",
        "value": rep["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "eager_ms_per_step": t["eager_ms"],
        "step_launch": "HIP graph replay of the three entry points (per-entry times and rooflines from the eager loop)",
        "settle": {"seconds": SETTLE_S, "steps": t["settle_steps"],
                   "note": "untimed steps right before each timed region, after the warmup steps: the GPU "
                           "returns to its steady clocks ~25 ms into a load after idling"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; drafts = greedy tokens corrupted with p=0.3)",
        "config": {"workload": wl.name, "B": len(x.pos), "k": wl.kmax, "rows": x.R,
                   "context": f"U{{{wl.ctx_lo}..{wl.ctx_hi}}}", "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "hidden": wl.H, "vocab": wl.V, "page": 16,
                   "kv_split_tokens": gdv.attn_split_tokens(x.page_table.shape[1])},
        **drafts_note,
        "emitted_tokens_per_s": rep["emitted_tokens_per_s"],
        "emitted_per_step": rep["emitted_per_step"],
        "accept_len_hist": rep["accept_len_hist"],
        "kernel_us": rep["kernel_us"],
        "kernel_us_median": rep["kernel_us_median"],
        "roofline": {"kernel": lm_call, "bound": lm["bound"],
                     "achieved": lm["GB/s"] if lm["bound"] == "hbm" else lm["TFLOP/s"],
                     "peak": HBM_PEAK_GBS if lm["bound"] == "hbm" else BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if lm["bound"] == "hbm" else "TFLOP/s", "frac": lm_frac,
                     "traffic": measured_traffic("lm_head_tile") if wl.name == "b16k4" else None,
                     "hbm_frac": lm["hbm_frac"], "mfma_frac": lm["mfma_frac"],
                     "algorithmic_bytes": lm["algorithmic_bytes"]},
        "attn_roofline": {"kernel": "spec_verify_attn", "bound": "hbm", "achieved": at["achieved"],
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": at["frac"],
                          "algorithmic_bytes": at["algorithmic_bytes"],
                          # the call's two kernels: the split kernel and the combine
                          "traffic": (None if wl.name != "b16k4" or measured_traffic("attn_kernel") is None
                                      or measured_traffic("attn_combine") is None
                                      else measured_traffic("attn_kernel") + measured_traffic("attn_combine"))},
        "cpu_baseline": cpu,
        **extras,
        "context": "pages' own figure: 6.5 ms per 16-row whole-model verify, RTX 5090 with CUDA graphs "
                   "(not comparable: whole model, other hardware)",
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
