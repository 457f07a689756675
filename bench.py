#!/usr/bin/env python3
"""Benchmark of the anchor-masked block-sparse cross-attention hot path on one GPU.

One step is one pass of the whole path over the 8192-query x 65536-token packed
context (Hq = 32, Hkv = 8, head_dim = 128, bf16), split into 64 chunks of 1024
tokens and planned onto 8 virtual devices ("bins"):

  1. chunk_cost   realised cost of each chunk (GPU, int64)
  2. lpt_plan     longest-processing-time-first plan with equal chunk counts (GPU; the
                  same plan as the host lpt_assign, so nothing returns to the host)
  3. per bin: context_gather of its chunks of K and V into its local buffer, and
     sparse_xattn_fwd (the own-block term on bin 0): partial O, lse; the bins
     alternate between two streams, each stream gathering its later bins right
     after its first forward, so one stream's gathers overlap the other's forward
  4. lse_combine  of the 8 partials
  5. sparse_xattn_bwd: delta pre-pass, then the dQ phase of every bin (accumulated,
     on a second stream) beside the dK/dV phase of every bin (bf16 dK, dV)

Throughput is useful attention FLOP/s: 4*d*Hq FLOP per allowed (query, key) pair
for the forward and 10*d*Hq for the backward, over the allowed pairs only
(context pairs from the cost kernel plus 16 own-block pairs per query).

Prints one JSON line.  The timed steps carry no HIP events (recording one costs GPU
time); the per-phase breakdown comes from the warm-up steps, which carry events
around every phase, and the dominant phase's roofline from its calls run alone after
the timed steps.  The CPU oracle is timed on a bounded sample of blocks of the same
workload.

`--combine P` times the P-way combine of the 8192-query view instead (every partial
live, and the empty pattern of the 524288-token workload on P bins; one JSON line).

`--dense KEYS` times the forward, dQ and dK/dV phases of one dense call instead
(8192 queries that may all read KEYS keys; one JSON line).

`--balance WORKLOAD` runs the per-bin balance study instead (one JSON line): every
bin's share of the context alone on the GPU under three plans (LPT on the pair cost,
LPT on a tile-granular cost, contiguous chunks), and how well per-chunk costs and a
dispatch model predict the per-bin kernel times.
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "useful attn TFLOP/s fwd+bwd, 8k q × 64k ctx bf16; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
WORKLOAD = "fwdbwd_bf16_8kq_64k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timers:
    """HIP events around phases on the current stream, grouped by phase name.

    `only` selects the phases that get events: None (none), "all", or one name.
    Events are created by `reserve` before they are recorded: creating them inside
    a timed region can stall the host for tens of milliseconds once the runtime
    grows its event pool, and the GPU would run dry meanwhile."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.only = None
        self.calls = {}   # phase name -> calls seen while counting
        self.pool = []

    def reserve(self, n):
        t = self.torch
        self.pool = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
                     for _ in range(n)]
        self.pool.reverse()

    def run(self, name, work, fn, launches=1, stream=None):
        """Run fn, with events on `stream` (default: the current stream) around it."""
        if self.only is None:
            self.calls[name] = self.calls.get(name, 0) + 1
            return fn()
        if self.only != "all" and self.only != name:
            return fn()
        if not self.pool:
            raise RuntimeError("Timers: more timed phases than reserved events")
        e0, e1 = self.pool.pop()
        e0.record(stream)
        out = fn()
        e1.record(stream)
        self.pending.append((name, work, launches, e0, e1))
        return out

    def summary(self):
        agg = {}
        for name, work, launches, e0, e1 in self.pending:
            ms = e0.elapsed_time(e1)
            a = agg.setdefault(name, {"ms": 0.0, "launches": 0, "work": 0.0, "calls": 0})
            a["ms"] += ms
            a["launches"] += launches
            a["work"] += work
            a["calls"] += 1
        return agg


def build_problem(torch, seed, split=False, inputs=None, bwd_schedule="overlap"):
    """Device buffers, plan buffers, streams and events of the benchmark step.
    ``inputs`` (a function of the workload and its metadata returning synth.Inputs
    over the whole context) replaces the default draw, for tests that run the step on
    other values."""
    from block_sparse_cross_anchor_amd import synth, sxattn

    w = synth.WORKLOADS[WORKLOAD]
    meta = synth.meta_for(w, seed)
    all_rows = np.arange(w.n_ctx)
    if inputs is None:
        inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(),
                                np.array([0], np.int32), np.array([w.n_ctx], np.int32),
                                with_dout=True)
    else:
        inp = inputs(w, meta)

    def dev(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    P = {
        "w": w, "meta": meta, "inp": inp, "all_rows": all_rows,
        "q": dev(inp.q), "k": dev(inp.k), "v": dev(inp.v), "ks": dev(inp.k_self),
        "vs": dev(inp.v_self), "do": dev(inp.dout),
        "anchor": torch.as_tensor(meta.anchor).cuda(),
        "start": torch.as_tensor(meta.sample_start).cuda(),
    }
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    P["chunk_gs"], P["chunk_gl"] = gs, gl
    n_q, hq, hkv, d, nb = w.n_q, w.hq, w.hkv, w.d, w.n_bin
    per_bin = w.n_chunk // nb
    n_loc = per_bin * w.chunk_size
    bf, f32 = torch.bfloat16, torch.float32
    P["k_loc"] = torch.empty((nb, n_loc, hkv, d), dtype=bf, device="cuda")
    P["v_loc"] = torch.empty_like(P["k_loc"])
    # key/value gradients in bf16 (summed in float32 inside the library, rounded once)
    P["dk_loc"] = torch.empty((nb, n_loc, hkv, d), dtype=bf, device="cuda")
    P["dv_loc"] = torch.empty_like(P["dk_loc"])
    P["dks"] = torch.empty(P["ks"].shape, dtype=bf, device="cuda")
    P["dvs"] = torch.empty_like(P["dks"])
    P["o_parts"] = torch.empty((nb, n_q, hq, d), dtype=bf, device="cuda")
    P["lse_parts"] = torch.empty((nb, n_q, hq), dtype=f32, device="cuda")
    P["o"] = torch.empty((n_q * hq, d), dtype=bf, device="cuda")
    P["lse"] = torch.empty((n_q * hq,), dtype=f32, device="cuda")
    P["delta"] = torch.empty((2, n_q, hq), dtype=f32, device="cuda")
    P["dq"] = torch.empty((n_q, hq, d), dtype=f32, device="cuda")
    P["cost"] = torch.empty((w.n_chunk,), dtype=torch.int64, device="cuda")
    # the device plan: every chunk's bin, every bin's load, and each bin's chunk list
    # (starts, lengths), which the gathers and attention calls of that bin read
    P["chunk_gs_d"] = torch.as_tensor(gs).cuda()
    P["chunk_gl_d"] = torch.as_tensor(gl).cuda()
    P["bin_of_d"] = torch.empty((w.n_chunk,), dtype=torch.int32, device="cuda")
    P["load_d"] = torch.empty((nb,), dtype=torch.int64, device="cuda")
    P["plan"] = torch.empty((2, nb, per_bin), dtype=torch.int32, device="cuda")
    P["plan_gs"], P["plan_gl"] = P["plan"][0], P["plan"][1]
    P["per_bin"], P["n_loc"] = per_bin, n_loc
    P["scale"] = 1.0 / math.sqrt(d)
    # The bins' gathers and forwards alternate between the current stream and a
    # second one (default priority), so one bin's forward overlaps the other
    # stream's gather and the tail of its forward.  Each stream has its own forward
    # workspace; the two events that fork and join the streams are created here,
    # outside any timed region.
    P["side_stream"] = torch.cuda.Stream()
    P["bwd_schedule"] = bwd_schedule
    # each bin's call metadata: views of the device plan, which every step rewrites
    P["metas"] = []
    for b in range(nb):
        m = sxattn.Meta.__new__(sxattn.Meta)
        m.anchor, m.sample_start = P["anchor"], P["start"]
        m.chunk_gstart, m.chunk_len = P["plan_gs"][b], P["plan_gl"][b]
        m.n_blk, m.n_chunk, m.n_loc = w.n_anchor, per_bin, n_loc
        P["metas"].append(m)
    P["live_rows"] = {}   # live partial rows of the combine, per plan
    P["ev_fork"] = torch.cuda.Event()
    P["ev_fork_dq"] = torch.cuda.Event()
    P["ev_join_dq"] = torch.cuda.Event()
    P["ev_join"] = torch.cuda.Event()
    # The dQ phase runs as two halves of the blocks, one per stream: blocks are
    # independent and the halves write disjoint dQ rows.  Each half has its own call
    # metadata, delta buffer (a call's delta planes are laid out for its own rows)
    # and workspace.
    lib = sxattn.load_library()
    half = w.n_anchor // 2
    P["dq_halves"] = []
    for b0, b1 in ((0, half), (half, w.n_anchor)):
        hm = []
        for b in range(nb):
            m = sxattn.Meta.__new__(sxattn.Meta)
            m.anchor, m.sample_start = P["anchor"][b0:b1], P["start"][b0:b1]
            m.chunk_gstart, m.chunk_len = P["plan_gs"][b], P["plan_gl"][b]
            m.n_blk, m.n_chunk, m.n_loc = b1 - b0, per_bin, n_loc
            hm.append(m)
        bws = int(lib.sparse_xattn_bwd_split_workspace_bytes(b1 - b0, n_loc, hq, hkv, d) if split
                  else lib.sparse_xattn_bwd_workspace_bytes(b1 - b0, n_loc, hq, hkv, d))
        P["dq_halves"].append({
            "tok": slice(16 * b0, 16 * b1), "metas": hm,
            "delta": torch.empty((2, 16 * (b1 - b0), hq), dtype=f32, device="cuda"),
            "ws": torch.empty((max(bws, 256),), dtype=torch.uint8, device="cuda")})
    bws = int(lib.sparse_xattn_bwd_split_workspace_bytes(w.n_anchor, n_loc, hq, hkv, d) if split
              else lib.sparse_xattn_bwd_workspace_bytes(w.n_anchor, n_loc, hq, hkv, d))
    P["bwd_ws"] = [torch.empty((max(bws, 256),), dtype=torch.uint8, device="cuda") for _ in range(2)]
    fws = int(lib.sparse_xattn_fwd_split_workspace_bytes(w.n_anchor, hq, hkv, d) if split
              else lib.sparse_xattn_fwd_workspace_bytes(w.n_anchor, hq, hkv))
    P["fwd_ws"] = [torch.empty((max(fws, 256),), dtype=torch.uint8, device="cuda") for _ in range(2)]
    # The same plan on the host, once: the GPU costs copied back and the host LPT.  The
    # step plans on the device; these host values only size the timers' work and the
    # reported fields (the metadata, hence the plan, is the same every step), and
    # check_device_plan() compares the device's plan with them after the timed steps.
    sxattn.chunk_cost(P["anchor"], P["start"], w.n_ctx, w.chunk_size, out=P["cost"])
    cost_np = P["cost"].cpu().numpy()
    bins, load = sxattn.lpt_assign(cost_np, nb)
    bins_np = bins.numpy()
    order = np.argsort(bins_np, kind="stable").reshape(nb, per_bin)   # chunks of each bin
    P["host_plan"] = (bins_np, load.numpy(), cost_np, order)
    return P


def plan(torch, P, T):
    """Steps 1 and 2 of the hot path, on the device: the cost of every chunk, then the
    LPT plan into the plan buffers that every later launch reads.  Nothing returns to
    the host, so the step is enqueued without waiting for the GPU."""
    from block_sparse_cross_anchor_amd import sxattn

    w = P["w"]
    T.run("chunk_cost", 8 * w.n_anchor + 8 * w.n_chunk,
          lambda: sxattn.chunk_cost(P["anchor"], P["start"], w.n_ctx, w.chunk_size, out=P["cost"]))
    T.run("lpt_plan", 8 * w.n_chunk + 8 * w.n_chunk + 8 * w.n_bin + 8 * w.n_chunk,
          lambda: sxattn.lpt_plan(P["cost"], P["chunk_gs_d"], P["chunk_gl_d"], w.n_bin,
                                  bin_of=P["bin_of_d"], load=P["load_d"], plan=P["plan"]))


def step(torch, P, T):
    """One pass of the hot path; returns the plan (bins, load, cost) and the allowed
    pairs of each bin, from the host copy of the plan.  With a captured graph
    (P["graph"]) the whole step is one replay of it."""
    bins_np, load, cost_np, order = P["host_plan"]
    if P.get("graph") is not None:
        P["graph"].replay()
        bin_pairs = [int(cost_np[order[b]].sum()) for b in range(P["w"].n_bin)]
    else:
        plan(torch, P, T)
        bin_pairs = post_plan(torch, P, T, bins_np, cost_np, order)
    return bins_np, load, cost_np, bin_pairs


def check_device_plan(torch, P):
    """The device plan of the last step equals the host plan (bins, loads, lists)."""
    bins_np, load, _, order = P["host_plan"]
    torch.cuda.synchronize()
    ok = (np.array_equal(P["bin_of_d"].cpu().numpy(), bins_np)
          and np.array_equal(P["load_d"].cpu().numpy(), load)
          and np.array_equal(P["plan"][0].cpu().numpy(), P["chunk_gs"][order])
          and np.array_equal(P["plan"][1].cpu().numpy(), P["chunk_gl"][order]))
    if not ok:
        raise RuntimeError("the device LPT plan differs from the host plan")


def capture_graph(torch, P):
    """Capture a whole step (costs, device plan, gathers, forwards, combine, delta,
    dQ and dK/dV phases on both streams) into one HIP graph.  The plan is computed on
    the device inside it, so one capture serves every step; the capture itself runs
    nothing."""
    bins_np, _, cost_np, order = P["host_plan"]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan(torch, P, _NoTimer())
        post_plan(torch, P, _NoTimer(), bins_np, cost_np, order)
    torch.cuda.synchronize()
    P["graph"] = g


class _NoTimer:
    def run(self, name, work, fn, launches=1, stream=None):
        return fn()


def post_plan(torch, P, T, bins_np, cost_np, order):
    """Steps 3 to 5 of the hot path, enqueued on the current stream and the side
    stream; returns the allowed context pairs of each bin."""
    from block_sparse_cross_anchor_amd import sxattn

    w = P["w"]
    nb, n_loc, d, hq = w.n_bin, P["n_loc"], w.d, w.hq
    scale = P["scale"]
    self_pairs = 16 * w.n_q
    metas = P["metas"]
    main, side = torch.cuda.current_stream(), P["side_stream"]
    fwd_pairs = int(cost_np.sum()) + self_pairs

    def gathers_and_forwards():
        # The side stream starts once bin 0's context is gathered (after the plan and
        # after everything the previous step queued on the current stream, which reads
        # the buffers the gathers rewrite), so the two streams run half a gather apart.
        # Each stream gathers its later bins right after its first forward, beside the
        # other stream's forward; the current stream continues once both are done.
        def gather(b):
            for src, dst in ((P["k"], P["k_loc"][b]), (P["v"], P["v_loc"][b])):
                sxattn.context_gather(src, P["plan_gs"][b], P["plan_gl"][b], n_loc, out=dst)

        for b in range(nb):
            with torch.cuda.stream(main if b % 2 == 0 else side):
                if b == 1:
                    side.wait_event(P["ev_fork"])
                if b < 2:
                    gather(b)
                if b == 0:
                    P["ev_fork"].record(main)
                sxattn.sparse_xattn_fwd(
                    P["q"], P["k_loc"][b], P["v_loc"][b], metas[b], scale,
                    P["ks"] if b == 0 else None, P["vs"] if b == 0 else None,
                    out=P["o_parts"][b], lse=P["lse_parts"][b], workspace=P["fwd_ws"][b % 2])
                if b < 2:  # the stream's later bins, beside the other stream's first forward
                    for b2 in range(b + 2, nb, 2):
                        gather(b2)
        P["ev_join"].record(side)
        main.wait_event(P["ev_join"])

    T.run("gather_fwd", 4.0 * d * hq * fwd_pairs, gathers_and_forwards, launches=nb)
    bin_pairs = [int(cost_np[order[b]].sum()) for b in range(nb)]   # after the launches
    rows = w.n_q * hq
    # the combine's algorithmic bytes: O rows of the live partials only (a partial row
    # is empty where the block's interval meets none of the bin's chunks, and the
    # kernel does not read it), every lse, and the merged output
    key = bins_np.tobytes()
    if key not in P["live_rows"]:
        meta = P["meta"]
        lo = meta.sample_start.astype(np.int64)[:, None]
        hi = meta.anchor.astype(np.int64)[:, None]
        cs = P["chunk_gs"].astype(np.int64)[order]                   # [nb, per_bin]
        ce = cs + P["chunk_gl"].astype(np.int64)[order]
        live = [np.any(np.maximum(lo, cs[b][None, :]) < np.minimum(hi, ce[b][None, :]), axis=1)
                for b in range(nb)]
        live[0][:] = True   # bin 0 carries the own-block term
        P["live_rows"][key] = int(sum(int(x.sum()) for x in live)) * 16 * hq
    live_rows = P["live_rows"][key]
    T.run("lse_combine", live_rows * d * 2 + nb * rows * 4 + rows * (d * 2 + 4),
          lambda: sxattn.lse_combine(P["o_parts"].view(nb, rows, d), P["lse_parts"].view(nb, rows),
                                     out=P["o"], lse_out=P["lse"]))
    o = P["o"].view(w.n_q, hq, d)
    lse = P["lse"].view(w.n_q, hq)
    halves = P["dq_halves"]

    def half_args(hf, b):
        t = hf["tok"]
        return (P["q"][t], P["k_loc"][b], P["v_loc"][b], hf["metas"][b], scale, o[t], P["do"][t],
                lse[t], P["dq"][t])

    def whole_delta():
        sxattn.sparse_xattn_bwd(P["q"], P["k_loc"][0], P["v_loc"][0], metas[0], scale, o, P["do"],
                                lse, P["dq"], delta_ws=P["delta"], dk=P["dk_loc"][0],
                                dv=P["dv_loc"][0], flags=sxattn.BWD_DELTA, workspace=None)

    def deltas():   # the whole rows (for dK/dV), then each dQ half's own
        whole_delta()
        for hf in halves:
            sxattn.sparse_xattn_bwd(*half_args(hf, 0), delta_ws=hf["delta"], dk=P["dk_loc"][0],
                                    dv=P["dv_loc"][0], flags=sxattn.BWD_DELTA, workspace=hf["ws"])

    sched = P["bwd_schedule"]
    if sched == "halves":
        T.run("delta", 2 * rows * (2 * d * 2 + 4), deltas, launches=3)
    else:
        T.run("delta", rows * (2 * d * 2 + 4 + 8), whole_delta, launches=1)
    all_pairs = sum(bin_pairs) + self_pairs

    def dq_halves():
        P["ev_fork_dq"].record(main)
        side.wait_event(P["ev_fork_dq"])
        for i, hf in enumerate(halves):
            t = hf["tok"]
            with torch.cuda.stream(main if i == 0 else side):
                for b in range(nb):
                    sxattn.sparse_xattn_bwd(
                        *half_args(hf, b), P["ks"][t] if b == 0 else None,
                        P["vs"][t] if b == 0 else None, delta_ws=hf["delta"], dk=P["dk_loc"][b],
                        dv=P["dv_loc"][b], dk_self=P["dks"][t], dv_self=P["dvs"][t],
                        flags=sxattn.BWD_DQ | (sxattn.BWD_DQ_OVERWRITE if b == 0 else 0),
                        workspace=hf["ws"])
        P["ev_join_dq"].record(side)
        main.wait_event(P["ev_join_dq"])

    def bwd(b, flags, ws):
        self_kv = (P["ks"], P["vs"]) if b == 0 else (None, None)
        sxattn.sparse_xattn_bwd(
            P["q"], P["k_loc"][b], P["v_loc"][b], metas[b], scale, o, P["do"], lse, P["dq"],
            self_kv[0], self_kv[1], delta_ws=P["delta"], dk=P["dk_loc"][b], dv=P["dv_loc"][b],
            dk_self=P["dks"], dv_self=P["dvs"], flags=flags, workspace=ws)

    # one workspace per stream: the dK/dV phase's on this stream, the dQ phase's on the
    # side stream when the two overlap
    ws_main, ws_side = P["bwd_ws"]

    def dq_bins(ws):
        for b in range(nb):
            bwd(b, sxattn.BWD_DQ | (sxattn.BWD_DQ_OVERWRITE if b == 0 else 0), ws)

    def dkdv_bins():
        for b in range(nb):
            bwd(b, sxattn.BWD_DKDV, ws_main)

    dq_work, dkdv_work = 6.0 * d * hq * all_pairs, 8.0 * d * hq * all_pairs
    # the dK/dV phase alone (same inputs and plan), for its roofline outside the step
    P["dkdv_phase"] = (dkdv_work, dkdv_bins)
    if sched == "halves":
        # dQ: both halves' bins on two streams (bin 0 overwrites a half's rows, the others
        # add); dK/dV: one group of nb launches on this stream
        T.run("bwd_dq", dq_work, dq_halves, launches=2 * nb)
        T.run("bwd_dkdv", dkdv_work, dkdv_bins, launches=nb)
    elif sched == "serial":
        T.run("bwd_dq", dq_work, lambda: dq_bins(ws_main), launches=nb)
        T.run("bwd_dkdv", dkdv_work, dkdv_bins, launches=nb)
    else:
        # overlap: the dQ phase of every bin on the side stream beside the dK/dV phase of
        # every bin on this stream (they write disjoint buffers and read the same inputs)
        P["ev_fork_dq"].record(main)
        side.wait_event(P["ev_fork_dq"])
        with torch.cuda.stream(side):
            T.run("bwd_dq", dq_work, lambda: dq_bins(ws_side), launches=nb, stream=side)
        T.run("bwd_dkdv", dkdv_work, dkdv_bins, launches=nb)
        P["ev_join_dq"].record(side)
        main.wait_event(P["ev_join_dq"])
    return bin_pairs


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_8kq_64k_8bins.md")
KERNEL_SOURCE = {"sparse_xattn_fwd": "attn_fwd.hip", "bwd_dq": "attn_bwd.hip", "bwd_dkdv": "attn_bwd.hip"}


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    or None when the summary is missing or the kernel's source changed since."""
    import hashlib

    src = KERNEL_SOURCE.get(kernel)
    if src is None or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = v
    path = os.path.join(ROOT, "block_sparse_cross_anchor_amd", "csrc", src)
    if vals.get(src) != hashlib.sha256(open(path, "rb").read()).hexdigest():
        return None
    v = vals.get(f"{kernel}_bytes_per_launch")
    return None if v is None else float(v)


def cpu_baseline(P, seconds):
    """The oracle, as it stands, on a bounded sample of blocks of the same workload:
    forward then backward of the sampled blocks over the whole context."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    w, meta, inp = P["w"], P["meta"], P["inp"]
    q, k, v = inp.q.f64, inp.k.f64, inp.v.f64
    ks, vs, do = inp.k_self.f64, inp.v_self.f64, inp.dout.f64
    gs, gl = np.array([0], np.int32), np.array([w.n_ctx], np.int32)
    order = np.random.default_rng(0).permutation(meta.n_blk)
    done, pairs, t0 = 0, 0, time.perf_counter()
    batch = 4
    while done < meta.n_blk and time.perf_counter() - t0 < seconds:
        blocks = np.sort(order[done:done + batch])
        rows = np.concatenate([np.arange(16 * b, 16 * b + 16) for b in blocks])
        a, s = meta.anchor[blocks], meta.sample_start[blocks]
        o, lse = oracle.sparse_xattn_fwd(q[rows], k, v, a, s, gs, gl, P["scale"], ks[rows], vs[rows])
        oracle.sparse_xattn_bwd(q[rows], k, v, o, do[rows], lse, a, s, gs, gl, P["scale"],
                                ks[rows], vs[rows])
        pairs += int(16 * ((a.astype(np.int64) - s).sum() + 16 * len(blocks)))
        done += len(blocks)
    el = time.perf_counter() - t0
    flop = 14.0 * w.d * w.hq * pairs
    return {"value": flop / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {meta.n_blk} blocks (random order, seed 0), forward+backward "
                      f"over the whole 65536-token context, numpy float64; {el:.1f} s, "
                      f"{pairs} allowed pairs per head"}


def tile_costs(meta, n_ctx, chunk_size, hq, hkv):
    """Per-chunk work at the kernels' own granularity, in (query token, key) slots, for
    the balance study.  The pair cost counts only allowed pairs; these count whole
    tiles, edge tiles included:
      fwd_tiles   64-key tiles (aligned to the chunk start) that a forward / dQ row
                  group visits: the tiles meeting [min sample start, max anchor) over
                  the group's blocks, times the group's tokens;
      blk_tiles   64-key tiles meeting each block's own interval, times 16;
      dkdv_tiles  256-key tiles meeting each block's interval, times 16.
    Also returns the forward's 64-key tile count per (row group, chunk)."""
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    cs = np.arange(0, n_ctx, chunk_size, dtype=np.int64)
    ce = np.minimum(cs + chunk_size, n_ctx)

    def tiles(lo_g, hi_g, tk):
        a = np.maximum(lo_g[:, None], cs[None, :])
        e = np.minimum(hi_g[:, None], ce[None, :])
        n = -(-(e - cs[None, :]) // tk) - (a - cs[None, :]) // tk
        return np.where(a < e, n, 0)

    tok = 256 // (hq // hkv)          # tokens of a 256-row group
    bpg = max(tok // 16, 1)           # blocks per row group
    ng = -(-meta.n_blk // bpg)
    pad = ng * bpg - meta.n_blk
    lo_r = np.concatenate([lo, np.full(pad, lo[-1])]).reshape(ng, bpg).min(1)
    hi_r = np.concatenate([hi, np.full(pad, hi[-1])]).reshape(ng, bpg).max(1)
    group_tiles = tiles(lo_r, hi_r, 64)
    return {"fwd_tiles": (tok * 64 * group_tiles).sum(0),
            "blk_tiles": (16 * 64 * tiles(lo, hi, 64)).sum(0),
            "dkdv_tiles": (16 * 256 * tiles(lo, hi, 256)).sum(0)}, group_tiles


def dispatch_makespan(job_tiles, n_cu, overhead):
    """Finish time, in tile times, of jobs (one per forward / dQ workgroup) handed out
    in the kernels' dispatch order (most tiles first) to the first free compute unit,
    one at a time per unit, each costing its tiles plus a fixed overhead."""
    import heapq

    free = [0.0] * n_cu
    for t in sorted(job_tiles, reverse=True):
        heapq.heappush(free, heapq.heappop(free) + t + overhead)
    return max(free)


def split_jobs(job_tiles, cap, merge):
    """Row-group jobs as a split-KV forward would run them: a job of t > cap tiles
    becomes ceil(t / cap) pieces of equal share, each also paying `merge` tiles for
    writing its partial output and its part of the merge."""
    out = []
    for t in job_tiles:
        s = max(1, -(-int(t) // cap))
        out += [t / s + (merge if s > 1 else 0)] * s
    return out


def _fit(x, y):
    """Least-squares line y = a + b x: (R^2, largest |residual| / y)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    A = np.stack([np.ones_like(x), x], 1)
    coef = np.linalg.lstsq(A, y, rcond=None)[0]
    res = y - A @ coef
    ss = float(((y - y.mean()) ** 2).sum())
    return (1.0 - float((res ** 2).sum()) / ss if ss > 0 else 1.0), float(np.abs(res / y).max())


def balance_study(torch, workload, seed, reps):
    """Each bin's share of the context run alone on the GPU, under the LPT plan on the
    pair cost, the LPT plan on the forward's tile cost and the contiguous plan (bin b
    = chunks [b n/P, (b+1) n/P)).  Prints one JSON line with the per-bin kernel times
    of every plan, the max-bin time of each, and how well each per-chunk cost
    predicts the per-bin kernel times."""
    from block_sparse_cross_anchor_amd import synth, sxattn

    w = synth.WORKLOADS[workload]
    if not w.n_bin:
        raise SystemExit(f"workload {workload} has no bins")
    meta = synth.meta_for(w, seed)
    log(f"drawing the {w.n_ctx}-token context ...")
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(),
                            np.array([0], np.int32), np.array([w.n_ctx], np.int32),
                            with_dout=True)

    def dev(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    q, k, v, ks, vs, do = (dev(t) for t in (inp.q, inp.k, inp.v, inp.k_self, inp.v_self, inp.dout))
    del inp
    anchor = torch.as_tensor(meta.anchor).cuda()
    start = torch.as_tensor(meta.sample_start).cuda()
    n_q, hq, hkv, d, nb = w.n_q, w.hq, w.hkv, w.d, w.n_bin
    per_bin = w.n_chunk // nb
    n_loc = per_bin * w.chunk_size
    scale = 1.0 / math.sqrt(d)
    gs_all, gl_all = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    cost = sxattn.chunk_cost(anchor, start, w.n_ctx, w.chunk_size).cpu().numpy()
    tc, group_tiles = tile_costs(meta, w.n_ctx, w.chunk_size, hq, hkv)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plans = {"lpt_pairs": sxattn.lpt_assign(cost, nb)[0].numpy(),
             "lpt_fwd_tiles": sxattn.lpt_assign(tc["fwd_tiles"], nb)[0].numpy(),
             "contiguous": np.arange(w.n_chunk, dtype=np.int32) // per_bin}
    bf, f32 = torch.bfloat16, torch.float32
    k_loc = torch.empty((n_loc, hkv, d), dtype=bf, device="cuda")
    v_loc = torch.empty_like(k_loc)
    dk = torch.empty((n_loc, hkv, d), dtype=bf, device="cuda")   # bf16 gradients, as in the step
    dv = torch.empty_like(dk)
    o_p = torch.empty((n_q, hq, d), dtype=bf, device="cuda")
    lse_p = torch.empty((n_q, hq), dtype=f32, device="cuda")
    dq = torch.empty((n_q, hq, d), dtype=f32, device="cuda")
    delta = torch.empty((2, n_q, hq), dtype=f32, device="cuda")

    def share(bins_np, b):
        chunks = np.flatnonzero(bins_np == b)
        gsb = torch.as_tensor(gs_all[chunks]).cuda()
        glb = torch.as_tensor(gl_all[chunks]).cuda()
        sxattn.context_gather(k, gsb, glb, n_loc, out=k_loc)
        sxattn.context_gather(v, gsb, glb, n_loc, out=v_loc)
        return sxattn.Meta(anchor, start, gsb, glb, n_loc=n_loc), chunks

    # combined O and lse of the whole pass (own-block term included), which every
    # backward share reads
    log("combined forward ...")
    o_parts = torch.empty((nb, n_q, hq, d), dtype=bf, device="cuda")
    lse_parts = torch.empty((nb, n_q, hq), dtype=f32, device="cuda")
    for b in range(nb):
        m, _ = share(plans["lpt_pairs"], b)
        sxattn.sparse_xattn_fwd(q, k_loc, v_loc, m, scale, ks if b == 0 else None,
                                vs if b == 0 else None, out=o_parts[b], lse=lse_parts[b])
    o, lse = sxattn.lse_combine(o_parts.view(nb, n_q * hq, d), lse_parts.view(nb, n_q * hq))
    del o_parts, lse_parts
    o, lse = o.view(n_q, hq, d), lse.view(n_q, hq)
    m0, _ = share(plans["lpt_pairs"], 0)
    sxattn.sparse_xattn_bwd(q, k_loc, v_loc, m0, scale, o, do, lse, dq, delta_ws=delta,
                            dk=dk, dv=dv, flags=sxattn.BWD_DELTA)
    phases = {
        "fwd": lambda m: sxattn.sparse_xattn_fwd(q, k_loc, v_loc, m, scale, out=o_p, lse=lse_p),
        "fwd_split": lambda m: sxattn.sparse_xattn_fwd(q, k_loc, v_loc, m, scale, out=o_p, lse=lse_p,
                                                       workspace="split"),
        "dq": lambda m: sxattn.sparse_xattn_bwd(q, k_loc, v_loc, m, scale, o, do, lse, dq,
                                                delta_ws=delta, dk=dk, dv=dv,
                                                flags=sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE),
        "dq_split": lambda m: sxattn.sparse_xattn_bwd(q, k_loc, v_loc, m, scale, o, do, lse, dq,
                                                      delta_ws=delta, dk=dk, dv=dv,
                                                      flags=sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE,
                                                      workspace="split"),
        "dkdv": lambda m: sxattn.sparse_xattn_bwd(q, k_loc, v_loc, m, scale, o, do, lse, dq,
                                                  delta_ws=delta, dk=dk, dv=dv,
                                                  flags=sxattn.BWD_DKDV),
    }
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(len(plans) * nb * len(phases))]
    preds = {"pairs": cost, **tc}
    out = {"study": "balance", "workload": workload, "seed": seed, "bins": nb,
           "chunks": w.n_chunk, "reps": reps, "plans": {}}
    rows = []   # (plan, bin, phase ms..., predictor loads..., forward jobs' tiles)
    i = 0
    for name, bins_np in plans.items():
        log(f"plan {name} ...")
        per = {ph: [] for ph in phases}
        loads = {pn: [] for pn in preds}
        for b in range(nb):
            m, chunks = share(bins_np, b)
            for pn, pv in preds.items():
                loads[pn].append(int(pv[chunks].sum()))
            for ph, fn in phases.items():
                fn(m)   # warm
                e0, e1 = ev[i]
                i += 1
                e0.record()
                for _ in range(reps):
                    fn(m)
                e1.record()
                per[ph].append((e0, e1))
        torch.cuda.synchronize()
        ms = {ph: [e0.elapsed_time(e1) / reps for e0, e1 in per[ph]] for ph in phases}
        tot = [sum(ms[ph][b] for ph in phases if not ph.endswith("_split")) for b in range(nb)]
        for b in range(nb):
            jobs = np.repeat(group_tiles[:, bins_np == b].sum(1), hkv)
            rows.append((name, b, {ph: ms[ph][b] for ph in phases}, tot[b],
                         {pn: loads[pn][b] for pn in preds}, jobs))
        # the same totals with the forward and dQ phases on the split schedule
        tot_split = [ms["fwd_split"][b] + ms["dq_split"][b] + ms["dkdv"][b] for b in range(nb)]
        out["plans"][name] = {
            "max_bin_ms": round(max(tot), 4), "mean_bin_ms": round(float(np.mean(tot)), 4),
            "max_bin_ms_split": round(max(tot_split), 4),
            "mean_bin_ms_split": round(float(np.mean(tot_split)), 4),
            "time_imbalance": round(max(tot) / float(np.mean(tot)) - 1, 4),
            "phase_max_ms": {ph: round(max(ms[ph]), 4) for ph in phases},
            "load_imbalance": {pn: round(max(loads[pn]) / float(np.mean(loads[pn])) - 1, 4)
                               for pn in preds},
            "per_bin_ms": [round(t, 4) for t in tot],
            "per_bin_phase_ms": {ph: [round(t, 4) for t in ms[ph]] for ph in phases},
        }
    out["contiguous_over_lpt_pairs"] = round(out["plans"]["contiguous"]["max_bin_ms"]
                                             / out["plans"]["lpt_pairs"]["max_bin_ms"], 3)
    fits = {}
    for ph in [ph for ph in phases if not ph.endswith("_split")] + ["total"]:
        y = [r[3] if ph == "total" else r[2][ph] for r in rows]
        fits[ph] = {}
        for pn in preds:
            r2, worst = _fit([r[4][pn] for r in rows], y)
            fits[ph][pn] = {"r2": round(r2, 4), "max_rel_residual": round(worst, 4)}
    # the dispatch model for the two row-group kernels, its overhead fitted on a grid
    for ph in ("fwd", "dq"):
        y = [r[2][ph] for r in rows]
        best = None
        for ov in range(0, 17):
            x = [dispatch_makespan(r[5], n_cu, ov) for r in rows]
            r2, worst = _fit(x, y)
            if best is None or r2 > best[0]:
                best = (r2, worst, ov)
        fits[ph]["dispatch_model"] = {"r2": round(best[0], 4), "max_rel_residual": round(best[1], 4),
                                      "overhead_tiles": best[2]}
    out["fits"] = fits
    # split-KV inside one call, under the fitted dispatch model: the slowest bin of the
    # LPT plan with long jobs split, over the same bin unsplit
    lpt_rows = [r for r in rows if r[0] == "lpt_pairs"]
    out["split_model"] = {}
    for ph in ("fwd", "dq"):
        ov = fits[ph]["dispatch_model"]["overhead_tiles"]
        base = max(dispatch_makespan(r[5], n_cu, ov) for r in lpt_rows)
        out["split_model"][ph] = {
            f"cap_{cap}": round(max(dispatch_makespan(split_jobs(r[5], cap, 1), n_cu, ov)
                                    for r in lpt_rows) / base, 3)
            for cap in (8, 16, 32, 64)}
    out["split_measured"] = {
        name: {ph: {"max_bin_ms": p["phase_max_ms"][ph],
                    "split_max_bin_ms": p["phase_max_ms"][ph + "_split"],
                    "ratio": round(p["phase_max_ms"][ph + "_split"] / p["phase_max_ms"][ph], 3),
                    "mean_ratio": round(sum(p["per_bin_phase_ms"][ph + "_split"])
                                        / sum(p["per_bin_phase_ms"][ph]), 3)}
               for ph in ("fwd", "dq")}
        for name, p in out["plans"].items()}
    out["split_model_note"] = ("modelled max-bin time of the LPT plan with every row-group "
                               "job over cap tiles split into equal pieces (each paying the "
                               "fitted overhead plus one tile for its partial and merge), relative to "
                               "no split; below 1 would favour splitting")
    out["fits_note"] = ("line fitted to the per-bin kernel time over every bin of every "
                        "plan, against each per-chunk cost summed over the bin's chunks; "
                        "dispatch_model: against the makespan of the forward's row-group jobs "
                        f"on {n_cu} compute units, each costing its tiles plus a fitted overhead")
    print(json.dumps(out), flush=True)


def dense_study(torch, n_keys, seed, reps):
    """Forward, dQ and dK/dV phases of one dense call: 8192 queries (512 blocks) that
    may all read every one of n_keys context keys (one chunk, no own-block term),
    Hq 32, Hkv 8, d 128, bf16.  Prints one JSON line with each phase's time per call
    (HIP events around `reps` back-to-back calls) and its rate at 4d, 6d and 8d FLOP
    per pair."""
    from block_sparse_cross_anchor_amd import synth, sxattn

    n_blk, hq, hkv, d = 512, 32, 8, 128
    n_q = 16 * n_blk
    meta = synth.Meta(np.array([n_keys], np.int64), np.array([0], np.int64),
                      np.full(n_blk, n_keys, np.int32), np.zeros(n_blk, np.int32), n_keys)
    gs, gl = np.array([0], np.int32), np.array([n_keys], np.int32)
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "bf16", 1.0 / math.sqrt(d), gs, gl,
                            self_block=False, with_dout=True)

    def dev(t):
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    dm = sxattn.Meta(meta.anchor, meta.sample_start, gs, gl)
    scale = 1.0 / math.sqrt(d)
    o, lse = sxattn.sparse_xattn_fwd(q, k, v, dm, scale)
    dq = torch.zeros((n_q, hq, d), dtype=torch.float32, device="cuda")
    delta = torch.empty((2, n_q, hq), dtype=torch.float32, device="cuda")
    dk = torch.empty((n_keys, hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    bwd = lambda flags: sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq, delta_ws=delta,
                                                dk=dk, dv=dv, flags=flags)
    bwd(sxattn.BWD_DELTA)
    phases = {"fwd": (4, lambda: sxattn.sparse_xattn_fwd(q, k, v, dm, scale, out=o, lse=lse)),
              "dq": (6, lambda: bwd(sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE)),
              "dkdv": (8, lambda: bwd(sxattn.BWD_DKDV))}
    out = {"study": "dense", "n_q": n_q, "n_keys": n_keys, "hq": hq, "hkv": hkv, "head_dim": d,
           "reps": reps}
    pairs = n_q * n_keys
    for name, (per_pair, fn) in phases.items():
        fn()   # warm
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4),
                     "TFLOP/s": round(per_pair * d * hq * pairs / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps(out), flush=True)


def combine_study(torch, n_parts, seed, reps):
    """lse_combine of n_parts bf16 partials for every row of the 8192-query view
    (8192 x 32 heads, d 128), the merge one device performs at context-parallel size
    n_parts.  Two cases: every partial live (lse ~ U(0, 10), O ~ N(0, 0.1^2)), and
    the empty pattern of the 524288-token workload planned onto n_parts bins (a
    partial is empty, lse = -inf, where the block's interval meets none of that bin's
    chunks; the kernel never reads such a partial's O).  Eight seeded partial sets are
    drawn and repeated across the n_parts slots.  Returns each case's time per call
    and its rate in algorithmic bytes (O rows of live partials, every lse, the
    output)."""
    from block_sparse_cross_anchor_amd import synth, sxattn

    w = synth.WORKLOADS["cp64_share_8kq_512k"]
    n_q, hq, d = w.n_q, w.hq, w.d
    rows = n_q * hq
    o_parts = torch.empty((n_parts, rows, d), dtype=torch.bfloat16, device="cuda")
    n_draw = min(8, n_parts)
    for i in range(n_draw):
        o_i, _ = synth.draw_partials(seed + 100 * i, 1, rows, d, "bf16")
        src = torch.from_numpy(o_i.bits.view(np.int16)).view(torch.bfloat16).cuda()[0]
        for p in range(i, n_parts, n_draw):
            o_parts[p].copy_(src)
        del o_i, src
    rng = np.random.default_rng(seed)
    lse_dense = torch.as_tensor(rng.uniform(0.0, 10.0, size=(n_parts, rows)).astype(np.float32)).cuda()
    # the real empty pattern: LPT plan of the 524288-token workload onto n_parts bins
    meta = synth.meta_for(w, 5)
    cost = sxattn.chunk_cost(torch.as_tensor(meta.anchor).cuda(),
                             torch.as_tensor(meta.sample_start).cuda(), w.n_ctx,
                             w.chunk_size).cpu()
    bins = sxattn.lpt_assign(cost, n_parts)[0].numpy()
    gs_all, gl_all = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    lo = meta.sample_start.astype(np.int64)[:, None]
    hi = meta.anchor.astype(np.int64)[:, None]
    cs = gs_all.astype(np.int64)[None, :]
    meets = np.maximum(lo, cs) < np.minimum(hi, cs + gl_all[None, :])       # [n_blk, n_chunk]
    live_blk = np.stack([meets[:, bins == p].any(1) for p in range(n_parts)])  # [P, n_blk]
    live_blk[0] = True   # the own-block term lives on bin 0: its partial is never empty
    live = np.repeat(live_blk, 16 * hq, axis=1)                             # [P, rows]
    lse_empty = lse_dense.clone()
    lse_empty[torch.as_tensor(~live).cuda()] = float("-inf")
    out_o = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    out_l = torch.empty((rows,), dtype=torch.float32, device="cuda")
    result = {"study": "combine", "parts": n_parts, "rows": rows, "head_dim": d, "dtype": "bf16",
              "reps": reps, "peak_GB/s": PEAK_HBM_GBS}
    for name, lse, live_rows in (("all_live", lse_dense, n_parts * rows),
                                 ("empty_pattern", lse_empty, int(live.sum()))):
        fn = lambda: sxattn.lse_combine(o_parts, lse, out=out_o, lse_out=out_l)
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = live_rows * d * 2 + n_parts * rows * 4 + rows * (d * 2 + 4)
        gbs = nbytes / (ms * 1e-3) / 1e9
        result[name] = {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                        "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                        "live_fraction": round(live_rows / (n_parts * rows), 4)}
    del o_parts, lse_dense, lse_empty, out_o, out_l
    torch.cuda.empty_cache()
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)  # at least 1
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", action="store_true",
                    help="run the step's forwards and dQ phases on the split schedule")
    ap.add_argument("--graph", action="store_true",
                    help="replay the launches after each step's plan upload from one captured "
                         "HIP graph instead of enqueuing them from the host")
    ap.add_argument("--bwd-schedule", choices=("halves", "serial", "overlap"), default="overlap",
                    help="backward phases of the step: dQ in two halves of the blocks on two "
                         "streams then dK/dV (halves); dQ then dK/dV on one stream (serial); "
                         "dQ on a second stream beside dK/dV (overlap)")
    ap.add_argument("--balance", metavar="WORKLOAD",
                    help="instead of the benchmark, the per-bin balance study of a workload "
                         "with bins (fwdbwd_bf16_8kq_64k or cp64_share_8kq_512k)")
    ap.add_argument("--reps", type=int, default=5,
                    help="launches per timed share (--balance) or phase (--dense)")
    ap.add_argument("--combine", type=int, metavar="P",
                    help="instead of the benchmark, the P-way lse_combine of the 8192-query view")
    ap.add_argument("--dense", type=int, metavar="KEYS",
                    help="instead of the benchmark, the dense 8192-query x KEYS call of each "
                         "attention phase")
    args = ap.parse_args()
    if args.warmup < 1 or args.steps < 1:
        ap.error("--steps and --warmup must be at least 1")
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the context; --gpus {args.gpus} is not "
              "supported (the multi-device path is design only, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from block_sparse_cross_anchor_amd import sxattn

    sxattn.load_library()
    torch.cuda.set_device(0)
    if args.balance:
        balance_study(torch, args.balance, args.seed, max(args.reps, 1))
        return
    if args.dense:
        dense_study(torch, args.dense, args.seed, max(args.reps, 1))
        return
    if args.combine:
        print(json.dumps(combine_study(torch, args.combine, args.seed, max(args.reps, 1))),
              flush=True)
        return
    log("building the synthetic workload ...")
    P = build_problem(torch, args.seed, split=args.split, bwd_schedule=args.bwd_schedule)
    w = P["w"]
    T = Timers(torch)
    log(f"warmup {args.warmup} steps ...")
    step(torch, P, T)   # counts the timed phases of one step
    per_step = dict(T.calls)
    if args.warmup > 1:   # the other warm-up steps give the per-phase breakdown
        T.reserve(sum(per_step.values()) * (args.warmup - 1))
        T.only = "all"
        for _ in range(args.warmup - 1):
            step(torch, P, T)
        torch.cuda.synchronize()
        per_kernel = T.summary()
        T.pending = []
    else:
        per_kernel = {}
    T.only = None
    if args.graph:
        log("capturing the step's launches after the plan upload into a HIP graph ...")
        capture_graph(torch, P)
        step(torch, P, T)   # first replay, untimed
    log(f"timing {args.steps} steps ...")
    gc.collect()
    gc.disable()   # no collector pause inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bins, load, cost, bin_pairs = step(torch, P, T)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gc.enable()
    check_device_plan(torch, P)
    ms_step = el * 1e3 / args.steps
    ctx_pairs = int(cost.sum())
    pairs = ctx_pairs + 16 * w.n_q
    flop = 14.0 * w.d * w.hq * pairs
    value = flop / (ms_step * 1e-3) / 1e12
    # Roofline of the dominant kernel: the step's dK/dV calls (count, scan, main and
    # fix-up kernels each) run alone right after the timed steps, with HIP events
    # around each call, on the same inputs and plan.  Inside the step they share the
    # GPU with the dQ phase on the second stream (and replay from the graph), so
    # their own time is measured here; the in-step figure from the warm-up breakdown
    # is kept beside it.
    reps = 5
    work, fn = P["dkdv_phase"]
    T2 = Timers(torch)
    T2.reserve(reps)
    T2.only = "all"
    torch.cuda.synchronize()
    for _ in range(reps):
        T2.run("bwd_dkdv", work, fn, launches=w.n_bin)
    torch.cuda.synchronize()
    a = T2.summary()["bwd_dkdv"]
    avg_ms = a["ms"] / a["launches"]
    achieved = a["work"] / a["launches"] / (avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": recorded_traffic("bwd_dkdv"),
                "kernel": "bwd_dkdv", "avg_launch_ms": round(avg_ms, 4),
                "launches_per_step": w.n_bin,
                "measured": f"HIP events around each of the step's {w.n_bin} dK/dV calls (count, "
                            f"scan, main and fix-up kernels), run alone {reps} times right after "
                            "the timed steps on the same inputs and plan"}
    if "bwd_dkdv" in per_kernel:
        k = per_kernel["bwd_dkdv"]
        ms_l = k["ms"] / k["launches"]
        ach = k["work"] / k["launches"] / (ms_l * 1e-3) / 1e12
        roofline["in_step"] = {"achieved": round(ach, 2), "frac": round(ach / peak, 4),
                               "avg_launch_ms": round(ms_l, 4),
                               "measured": "the same calls inside the warm-up steps (eager, with "
                                           "events around every phase)"}
    kernels = {}   # from the warm-up steps with events around every phase
    n_bd = max(args.warmup - 1, 1)
    for n, k in per_kernel.items():
        mf = n in ("gather_fwd", "bwd_dq", "bwd_dkdv")
        rate = k["work"] / (k["ms"] * 1e-3) / (1e12 if mf else 1e9)
        kernels[n] = {"ms_per_step": round(k["ms"] / n_bd, 4),
                      ("TFLOP/s" if mf else "GB/s"): round(rate, 1)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "n_q": w.n_q, "n_ctx": w.n_ctx, "hq": w.hq,
                   "hkv": w.hkv, "head_dim": w.d, "block": 16, "chunks": w.n_chunk,
                   "chunk_size": w.chunk_size, "bins": w.n_bin, "seed": args.seed,
                   "row_group_schedule": "split" if args.split else "ranked",
                   "bwd_schedule": args.bwd_schedule, "graph": args.graph,
                   "allowed_pairs_per_head": pairs, "pct_of_bf16_peak": round(
                       100 * value / PEAK_BF16_TFLOPS, 2),
                   "lpt_imbalance": round(float(load.max() / load.mean() - 1), 5)},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": f"per-phase times from {n_bd} warm-up steps with events around every phase; "
                        "gather_fwd is the bins' context gathers and forwards on two streams, its "
                        "rate the forward's FLOP over that span; " + {
                            "halves": "bwd_dq runs two halves of the query blocks on two streams",
                            "serial": "bwd_dq then bwd_dkdv on one stream",
                            "overlap": "bwd_dq runs on a second stream beside bwd_dkdv, so their "
                                       "spans overlap"}[args.bwd_schedule],
    }
    # the combine one device performs at context-parallel size 64 (the 8192-query view,
    # 64 bf16 partials), every partial live and with the real empty pattern
    log("timing the 64-way combine of the 8192-query view ...")
    comb = combine_study(torch, 64, 5, 10)
    out["combine_64way"] = {
        "all_live": comb["all_live"], "empty_pattern": comb["empty_pattern"],
        "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "note": "lse_combine of 64 bf16 partials of all 262144 query rows (d 128), HIP events "
                "around 10 back-to-back calls; bytes are the O rows of live partials, every "
                "lse and the merged output"}
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s ...")
        out["cpu_baseline"] = cpu_baseline(P, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
