"""The benchmark's own step, checked against the oracle and against closed forms.

One pass of the hot path on the 8192-query x 65536-token workload (Hq 32, Hkv 8,
d 128, bf16) in exactly the launch configuration the benchmark times: chunk costs,
the LPT plan onto 8 bins, each bin's gather and forward (the bins alternating
between two streams), the 8-way combine, the delta pre-pass, the dQ phase of every
bin (accumulated, on a second stream) beside the load-balanced dK/dV phase of every
bin.

* Values ~ N(0, 1)/sqrt(d) (the workload's own): sampled outputs against the oracle,
  which evaluates each of them from the inputs alone (its backward consumes its own
  merged forward): merged O and lse of sampled blocks; dQ and the own-block dK, dV
  of sampled blocks; dK, dV of lightly read 64-key windows of three bins; and dK, dV
  of the most heavily read windows -- the first keys of one whole sample, read by
  every block of that sample, which the dK/dV schedule splits across workgroups
  and adds up in its fix-up pass -- plus windows spread over the rest of that sample
  (in whichever bins hold them).
* Values ~ N(0, 1) (sharp attention): the same sampled comparisons.
* Mask-boundary probe (Q = 0, one-hot values; tests/probe.py): every output of the
  step against its closed form -- O and lse of all 262144 query rows, dV of all
  65536 keys, dK = 0, dQ of all rows, own-block dK, dV.
"""

import math

import numpy as np
import pytest
import torch

import bench
import oracle
import probe
from block_sparse_cross_anchor_amd import synth
from helpers import (assert_lse_close, dkdv_split_tiles, host64, pick_windows, readers,
                     reader_pairs, rel_frob, sub_blocks, token_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SEED = 3


class _Untimed:
    def run(self, name, work, fn, launches=1, stream=None):
        return fn()


def _run_step(inputs=None):
    P = bench.build_problem(torch, SEED, inputs=inputs)
    bench.step(torch, P, _Untimed())
    torch.cuda.synchronize()
    return P


def _bin_chunks(P, b):
    return P["plan_gs"][b].cpu().numpy(), P["plan_gl"][b].cpu().numpy()


def _locate(P, g0):
    """(bin, local row) of global position g0 under the step's plan."""
    for b in range(P["w"].n_bin):
        gs, gl = _bin_chunks(P, b)
        off = 0
        for s, n in zip(gs, gl):
            if s <= g0 < s + n:
                return b, off + g0 - int(s)
            off += int(n)
    raise AssertionError(g0)


def _sample_windows(P, meta, budget):
    """The sample with the most blocks whose own allowed pairs stay within the budget;
    its first 16 windows of 64 keys (from the one holding the sample start) and one
    window per further 1024 keys.  Returns (sample, [(bin, local row, g0, readers)])."""
    blocks_of = np.searchsorted(meta.offsets, meta.sample_start, "right") - 1
    best = None
    for s in range(len(meta.lengths)):
        bl = np.flatnonzero(blocks_of == s)
        if bl.size and reader_pairs(meta, bl) <= budget and (best is None or bl.size > best[1]):
            best = (s, bl.size)
    s = best[0]
    start, end = int(meta.offsets[s]), int(meta.offsets[s] + meta.lengths[s])
    gpos = [start // 64 * 64 + 64 * i for i in range(16)]
    gpos += list(range(start // 64 * 64 + 1024, end - 64, 1024))
    out = []
    for g0 in gpos:
        if g0 + 64 > end or g0 // 1024 != (g0 + 63) // 1024:
            continue
        b, l0 = _locate(P, g0)
        out.append((b, l0, g0, readers(meta, g0, g0 + 64)))
    return s, out


def _check_sampled(P, rng_seed, heavy):
    w, meta, inp = P["w"], P["meta"], P["inp"]
    n_q, hq, d = w.n_q, w.hq, w.d
    scale = P["scale"]
    gs_all, gl_all = np.array([0], np.int32), np.array([w.n_ctx], np.int32)
    q64, k64, v64, do64 = inp.q.f64, inp.k.f64, inp.v.f64, inp.dout.f64
    ks64, vs64 = inp.k_self.f64, inp.v_self.f64
    o64 = host64(P["o"].view(n_q, hq, d))
    lse64 = host64(P["lse"].view(n_q, hq))

    rng = np.random.default_rng(rng_seed)
    starts = np.flatnonzero(np.diff(meta.sample_start) != 0) + 1  # first block of each sample
    blocks = np.unique(np.concatenate([[0, meta.n_blk - 1], starts[:3], starts[:3] - 1,
                                       rng.integers(0, meta.n_blk, 4)]))
    sub = sub_blocks(meta, blocks)
    rows = token_rows(blocks)

    # merged forward
    ro, rl = oracle.sparse_xattn_fwd(q64[rows], k64, v64, sub.anchor, sub.sample_start,
                                     gs_all, gl_all, scale, ks64[rows], vs64[rows])
    assert np.abs(o64[rows] - ro).max() <= 2e-2
    assert rel_frob(o64[rows], ro) <= 1e-2
    assert_lse_close(lse64[rows], rl, 1e-3)

    # dQ and own-block dK, dV of the sampled blocks, from the oracle's merged forward
    r = oracle.sparse_xattn_bwd(q64[rows], k64, v64, ro, do64[rows], rl,
                                sub.anchor, sub.sample_start, gs_all, gl_all, scale,
                                ks64[rows], vs64[rows])
    assert rel_frob(host64(P["dq"])[rows], r[0]) <= 3e-2
    assert rel_frob(host64(P["dks"])[rows], r[3]) <= 3e-2
    assert rel_frob(host64(P["dvs"])[rows], r[4]) <= 3e-2

    # dK, dV of local key windows (local row <-> global position through the plan):
    # a one-window oracle call over the blocks that read it, fed by the oracle's
    # forward of those blocks
    windows = []
    for b in (0, 3, 7):
        gsb, glb = _bin_chunks(P, b)
        windows += [(b, l0, g0, rd) for l0, g0, rd in pick_windows(meta, gsb, glb, rng, 2, 24)]
    n_light = len(windows)
    assert n_light >= 4
    sample = None
    if heavy:
        sample, hw = _sample_windows(P, meta, 1.2e7)
        windows += hw
    need = np.unique(np.concatenate([rd for _, _, _, rd in windows]))
    nrows = token_rows(need)
    sub_n = sub_blocks(meta, need)
    ro_n, rl_n = oracle.sparse_xattn_fwd(q64[nrows], k64, v64, sub_n.anchor, sub_n.sample_start,
                                         gs_all, gl_all, scale, ks64[nrows], vs64[nrows])
    pos = {int(x): i for i, x in enumerate(need)}
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    split_checked = 0
    for i, (b, l0, g0, rd) in enumerate(windows):
        wr = np.concatenate([np.arange(16 * pos[int(x)], 16 * pos[int(x)] + 16) for x in rd])
        sub_r = sub_blocks(meta, rd)
        g1, l1 = np.array([g0], np.int32), np.array([64], np.int32)
        rr = oracle.sparse_xattn_bwd(q64[token_rows(rd)], k64[g0:g0 + 64], v64[g0:g0 + 64],
                                     ro_n[wr], do64[token_rows(rd)], rl_n[wr], sub_r.anchor,
                                     sub_r.sample_start, g1, l1, scale)
        got_k = host64(P["dk_loc"][b][l0:l0 + 64])
        got_v = host64(P["dv_loc"][b][l0:l0 + 64])
        assert rel_frob(got_k, rr[1]) <= 3e-2, (b, l0, g0, rd.size)
        assert rel_frob(got_v, rr[2]) <= 3e-2, (b, l0, g0, rd.size)
        if i >= n_light:
            gsb, glb = _bin_chunks(P, b)
            shares = dkdv_split_tiles(meta, gsb, glb, hq, w.hkv, n_cu, b == 0)
            split_checked += int(shares[l0 // 256] >= 2)
    if heavy:
        blocks_of = np.searchsorted(meta.offsets, meta.sample_start, "right") - 1
        nb_s = int(np.sum(blocks_of == sample))
        # the window holding the sample start is read by every block of the sample
        assert windows[n_light][3].size >= nb_s and nb_s >= 24
        assert len(windows) - n_light >= 12
        assert split_checked >= 4, split_checked   # tiles split across workgroups


def test_benchmark_step_sampled_against_oracle():
    P = _run_step()
    _check_sampled(P, 7, heavy=True)


def test_benchmark_step_sharp_values_sampled():
    """The same step with Q, K, V, k_self, v_self ~ N(0, 1): sharp attention, where
    a wrong mask or a dropped key moves the outputs far beyond the bounds."""
    def sharp(w, meta):
        return synth.draw_inputs(SEED, meta, w.hq, w.hkv, w.d, "bf16", 1.0,
                                 np.array([0], np.int32), np.array([w.n_ctx], np.int32),
                                 with_dout=True)
    P = _run_step(sharp)
    _check_sampled(P, 8, heavy=False)


def test_benchmark_step_boundary_probe_all_outputs():
    """Q = 0 with one-hot probe values: every output of the step against its closed
    form (tests/probe.py, itself pinned against the oracle on the CPU)."""
    def probe_inputs(w, meta):
        return probe.inputs(SEED, meta, w.hq, w.hkv, w.d, np.array([0], np.int32),
                            np.array([w.n_ctx], np.int32), w.chunk_size)
    P = _run_step(probe_inputs)
    w, meta, inp = P["w"], P["meta"], P["inp"]
    n_q, hq, hkv, d = w.n_q, w.hq, w.hkv, w.d
    gs_all, gl_all = np.array([0], np.int32), np.array([w.n_ctx], np.int32)
    n_b, hits = probe.forward(meta, gs_all, gl_all, w.chunk_size, SEED)
    o = host64(P["o"].view(n_q, hq, d))
    lse = host64(P["lse"].view(n_q, hq))
    want = np.repeat(hits / n_b[:, None], 16, axis=0)[:, None, :]          # [n_q, 1, cols]
    err = np.abs(o[..., :probe.N_COLS] - want)
    assert np.all(err <= 2 ** -7 * want + 1e-6), float(err.max())
    assert np.all(o[..., probe.N_COLS:] == 0)
    np.testing.assert_allclose(lse, np.repeat(np.log(n_b), 16)[:, None] * np.ones((1, hq)),
                               rtol=0, atol=1e-5)
    # dV of every key of every bin, per 256-key tile; dK = 0
    dv_all = probe.dv_context(meta, inp, gs_all, gl_all, hq, hkv)
    for b in range(w.n_bin):
        gsb, glb = _bin_chunks(P, b)
        gpos = synth.chunk_rows(gsb, glb)
        got = host64(P["dv_loc"][b])
        want_v = dv_all[gpos]
        for t0 in range(0, gpos.size, 256):
            assert rel_frob(got[t0:t0 + 256], want_v[t0:t0 + 256]) <= 1e-2, (b, t0)
        assert torch.count_nonzero(P["dk_loc"][b]).item() == 0
    assert rel_frob(host64(P["dvs"]), probe.dv_self(meta, inp, gs_all, gl_all, hq, hkv)) <= 1e-2
    assert torch.count_nonzero(P["dks"]).item() == 0
    # dQ of every row, per block
    want_q = probe.dq(meta, inp, gs_all, gl_all, hq, hkv, P["scale"], w.chunk_size, SEED)
    got_q = host64(P["dq"])
    assert rel_frob(got_q, want_q) <= 1e-2
    for b in range(meta.n_blk):
        r = slice(16 * b, 16 * b + 16)
        assert rel_frob(got_q[r], want_q[r]) <= 3e-2, b


def test_benchmark_step_graph_replays_match_eager():
    """The benchmark replays the launches after the plan upload from one captured HIP
    graph.  Every replay, with eager work between them (the plan of the next step, and
    all outputs overwritten with NaN), must reproduce the eager step bit for bit: the
    kernels are deterministic and read the plan from the device buffers each step
    rewrites."""
    P = bench.build_problem(torch, SEED)
    bench.step(torch, P, _Untimed())
    torch.cuda.synchronize()
    names = ("o_parts", "lse_parts", "o", "lse", "delta", "dq", "dk_loc", "dv_loc", "dks", "dvs")
    want = {k: P[k].clone() for k in names}
    bench.capture_graph(torch, P)
    for rep in range(3):
        for k in names:
            P[k].fill_(float("nan"))
        torch.cuda.synchronize()
        bench.step(torch, P, _Untimed())
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(P[k], want[k]), (rep, k)
