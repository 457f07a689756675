#!/usr/bin/env python3
"""Benchmark of the anchor-masked block-sparse cross-attention hot path on one GPU.

One step is one pass of the whole path over the 8192-query x 65536-token packed
context (Hq = 32, Hkv = 8, head_dim = 128, bf16), split into 64 chunks of 1024
tokens and planned onto 8 virtual devices ("bins"):

  1. chunk_cost   realised cost of each chunk (GPU, int64), copied to the host
  2. lpt_assign   longest-processing-time-first plan with equal chunk counts (host)
  3. per bin: context_gather of its chunks of K and V into its local buffer, then
     sparse_xattn_fwd (the own-block term on bin 0): partial O, lse
  4. lse_combine  of the 8 partials
  5. sparse_xattn_bwd: delta pre-pass, then the dQ phase of every bin (accumulated)
     and the dK/dV phase of every bin

Throughput is useful attention FLOP/s: 4*d*Hq FLOP per allowed (query, key) pair
for the forward and 10*d*Hq for the backward, over the allowed pairs only
(context pairs from the cost kernel plus 16 own-block pairs per query).

Prints one JSON line.  The timed steps carry HIP events only around the dominant
phase (one pair per step around its 8 launches): recording an event costs GPU time,
so events around every launch would slow the step they measure.  The per-phase
breakdown comes from the warm-up steps, which carry events around every phase.  The
CPU oracle is timed on a bounded sample of blocks of the same workload.
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
WORKLOAD = "fwd_bf16_8kq_64k"


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

    def run(self, name, work, fn, launches=1):
        if self.only is None:
            self.calls[name] = self.calls.get(name, 0) + 1
            return fn()
        if self.only != "all" and self.only != name:
            return fn()
        if not self.pool:
            raise RuntimeError("Timers: more timed phases than reserved events")
        e0, e1 = self.pool.pop()
        e0.record()
        out = fn()
        e1.record()
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


def build_problem(torch, seed):
    from block_sparse_cross_anchor_amd import synth, sxattn

    w = synth.WORKLOADS[WORKLOAD]
    meta = synth.meta_for(w, seed)
    all_rows = np.arange(w.n_ctx)
    std = w.std()
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", std,
                            np.array([0], np.int32), np.array([w.n_ctx], np.int32),
                            with_dout=True)

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
    P["dk_loc"] = torch.empty((nb, n_loc, hkv, d), dtype=f32, device="cuda")
    P["dv_loc"] = torch.empty_like(P["dk_loc"])
    P["dks"] = torch.empty(P["ks"].shape, dtype=f32, device="cuda")
    P["dvs"] = torch.empty_like(P["dks"])
    P["o_parts"] = torch.empty((nb, n_q, hq, d), dtype=bf, device="cuda")
    P["lse_parts"] = torch.empty((nb, n_q, hq), dtype=f32, device="cuda")
    P["o"] = torch.empty((n_q * hq, d), dtype=bf, device="cuda")
    P["lse"] = torch.empty((n_q * hq,), dtype=f32, device="cuda")
    P["delta"] = torch.empty((2, n_q, hq), dtype=f32, device="cuda")
    P["dq"] = torch.empty((n_q, hq, d), dtype=f32, device="cuda")
    P["cost"] = torch.empty((w.n_chunk,), dtype=torch.int64, device="cuda")
    # the plan's host side in allocated pinned memory: one D2H of the costs and one
    # H2D of the packed plan per step, neither through a staging copy
    P["cost_h"] = torch.empty((w.n_chunk,), dtype=torch.int64, pin_memory=True)
    P["plan_h"] = torch.empty((2, nb, per_bin), dtype=torch.int32, pin_memory=True)
    P["plan"] = torch.empty((2, nb, per_bin), dtype=torch.int32, device="cuda")
    P["plan_gs"], P["plan_gl"] = P["plan"][0], P["plan"][1]
    P["per_bin"], P["n_loc"] = per_bin, n_loc
    P["scale"] = 1.0 / math.sqrt(d)
    return P


def step(torch, P, T):
    """One pass of the hot path; returns the host-side plan (bins, load, cost)."""
    from block_sparse_cross_anchor_amd import sxattn

    w = P["w"]
    nb, per_bin, n_loc, d, hq = w.n_bin, P["per_bin"], P["n_loc"], w.d, w.hq
    scale = P["scale"]
    T.run("chunk_cost", 8 * w.n_anchor + 8 * w.n_chunk,
          lambda: sxattn.chunk_cost(P["anchor"], P["start"], w.n_ctx, w.chunk_size, out=P["cost"]))
    P["cost_h"].copy_(P["cost"])                            # device -> host, synchronises
    cost = P["cost_h"]
    bins, load = sxattn.lpt_assign(cost, nb)                # host planner
    bins_np = bins.numpy()
    order = np.argsort(bins_np, kind="stable").reshape(nb, per_bin)   # chunks of each bin
    plan_h = P["plan_h"].numpy()
    plan_h[0] = P["chunk_gs"][order]
    plan_h[1] = P["chunk_gl"][order]
    # the host buffer is next written after the next step's cost copy, which waits
    # for this copy
    P["plan"].copy_(P["plan_h"], non_blocking=True)
    cost_np = cost.numpy()
    bin_pairs = [int(cost_np[order[b]].sum()) for b in range(nb)]
    self_pairs = 16 * w.n_q
    row_bytes = w.hkv * d * 2
    metas = []
    for b in range(nb):
        gsb, glb = P["plan_gs"][b], P["plan_gl"][b]
        for src, dst in ((P["k"], P["k_loc"][b]), (P["v"], P["v_loc"][b])):
            T.run("context_gather", 2 * n_loc * row_bytes,
                  lambda src=src, dst=dst: sxattn.context_gather(src, gsb, glb, n_loc, out=dst))
        m = sxattn.Meta.__new__(sxattn.Meta)
        m.anchor, m.sample_start, m.chunk_gstart, m.chunk_len = P["anchor"], P["start"], gsb, glb
        m.n_blk, m.n_chunk, m.n_loc = w.n_anchor, per_bin, n_loc
        metas.append(m)
        pairs = bin_pairs[b] + (self_pairs if b == 0 else 0)
        T.run("sparse_xattn_fwd", 4.0 * d * hq * pairs,
              lambda b=b: sxattn.sparse_xattn_fwd(
                  P["q"], P["k_loc"][b], P["v_loc"][b], metas[b], scale,
                  P["ks"] if b == 0 else None, P["vs"] if b == 0 else None,
                  out=P["o_parts"][b], lse=P["lse_parts"][b]))
    rows = w.n_q * hq
    T.run("lse_combine", nb * rows * (d * 2 + 4) + rows * (d * 2 + 4),
          lambda: sxattn.lse_combine(P["o_parts"].view(nb, rows, d), P["lse_parts"].view(nb, rows),
                                     out=P["o"], lse_out=P["lse"]))
    o = P["o"].view(w.n_q, hq, d)
    lse = P["lse"].view(w.n_q, hq)
    T.run("delta", rows * (2 * d * 2 + 4),
          lambda: sxattn.sparse_xattn_bwd(P["q"], P["k_loc"][0], P["v_loc"][0], metas[0], scale, o,
                                          P["do"], lse, P["dq"], delta_ws=P["delta"],
                                          dk=P["dk_loc"][0], dv=P["dv_loc"][0],
                                          flags=sxattn.BWD_DELTA))
    all_pairs = sum(bin_pairs) + self_pairs

    def bwd(b, flags):
        self_kv = (P["ks"], P["vs"]) if b == 0 else (None, None)
        sxattn.sparse_xattn_bwd(
            P["q"], P["k_loc"][b], P["v_loc"][b], metas[b], scale, o, P["do"], lse, P["dq"],
            self_kv[0], self_kv[1], delta_ws=P["delta"], dk=P["dk_loc"][b], dv=P["dv_loc"][b],
            dk_self=P["dks"], dv_self=P["dvs"], flags=flags)

    # each phase as one group of nb launches (bin 0 overwrites dQ, the others add)
    T.run("bwd_dq", 6.0 * d * hq * all_pairs,
          lambda: [bwd(b, sxattn.BWD_DQ | (sxattn.BWD_DQ_OVERWRITE if b == 0 else 0)) for b in range(nb)],
          launches=nb)
    T.run("bwd_dkdv", 8.0 * d * hq * all_pairs,
          lambda: [bwd(b, sxattn.BWD_DKDV) for b in range(nb)], launches=nb)
    return bins_np, load.numpy(), cost_np, bin_pairs


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)  # at least 1
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    log("building the synthetic workload ...")
    P = build_problem(torch, args.seed)
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
    # the dominant phase: the most time per step in the breakdown (the backward's
    # dK/dV phase when there is no breakdown)
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms"]) if per_kernel else "bwd_dkdv"
    T.reserve(per_step[dom] * args.steps)
    T.only = dom
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
    ms_step = el * 1e3 / args.steps
    ctx_pairs = int(cost.sum())
    pairs = ctx_pairs + 16 * w.n_q
    flop = 14.0 * w.d * w.hq * pairs
    value = flop / (ms_step * 1e-3) / 1e12
    a = T.summary()[dom]
    avg_ms = a["ms"] / a["launches"]
    work_per_launch = a["work"] / a["launches"]
    is_mfma = dom in ("sparse_xattn_fwd", "bwd_dq", "bwd_dkdv")
    achieved = work_per_launch / (avg_ms * 1e-3) / (1e12 if is_mfma else 1e9)
    peak = PEAK_BF16_TFLOPS if is_mfma else PEAK_HBM_GBS
    roofline = {"bound": "mfma" if is_mfma else "hbm", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s" if is_mfma else "GB/s",
                "frac": round(achieved / peak, 4), "traffic": recorded_traffic(dom), "kernel": dom,
                "avg_launch_ms": round(avg_ms, 4), "launches_per_step": a["launches"] // args.steps}
    kernels = {}   # from the warm-up steps with events around every phase
    n_bd = max(args.warmup - 1, 1)
    for n, k in per_kernel.items():
        mf = n in ("sparse_xattn_fwd", "bwd_dq", "bwd_dkdv")
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
                   "allowed_pairs_per_head": pairs, "pct_of_bf16_peak": round(
                       100 * value / PEAK_BF16_TFLOPS, 2),
                   "lpt_imbalance": round(float(load.max() / load.mean() - 1), 5)},
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": f"per-phase times from {n_bd} warm-up steps with events around every phase",
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_seconds:.0f} s ...")
        out["cpu_baseline"] = cpu_baseline(P, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
