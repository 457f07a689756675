"""The benchmark's own step, checked against the oracle on sampled outputs.

One pass of the hot path on the 8192-query x 65536-token workload (Hq 32, Hkv 8,
d 128, bf16) in exactly the launch configuration the benchmark times: chunk costs,
the LPT plan onto 8 bins, each bin's gather and forward (the bins alternating
between two streams), the 8-way combine, the delta pre-pass, the dQ phase of every
bin (accumulated; two halves of the query blocks on two streams) and the
load-balanced dK/dV phase of every bin.  Sampled outputs are compared with the
oracle, which evaluates each of them from the inputs alone (its backward consumes
its own merged forward):
  * merged O and lse of sampled blocks (all of their allowed keys),
  * dQ and the own-block dK, dV of sampled blocks,
  * dK, dV of 64-key windows of three bins' local buffers (windows read by at most
    24 blocks, so that the oracle's forward of those blocks stays small), mapped back
    to their global positions through the plan.
"""

import math

import numpy as np
import pytest
import torch

import bench
import oracle
from helpers import assert_lse_close, host64, pick_windows, rel_frob, sub_blocks, token_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


class _Untimed:
    def run(self, name, work, fn, launches=1, stream=None):
        return fn()


def test_benchmark_step_sampled_against_oracle():
    P = bench.build_problem(torch, 3)
    bins, load, cost, bin_pairs = bench.step(torch, P, _Untimed())
    torch.cuda.synchronize()
    w, meta, inp = P["w"], P["meta"], P["inp"]
    n_q, hq, d = w.n_q, w.hq, w.d
    scale = P["scale"]
    gs_all, gl_all = np.array([0], np.int32), np.array([w.n_ctx], np.int32)
    q64, k64, v64, do64 = inp.q.f64, inp.k.f64, inp.v.f64, inp.dout.f64
    ks64, vs64 = inp.k_self.f64, inp.v_self.f64
    o64 = host64(P["o"].view(n_q, hq, d))
    lse64 = host64(P["lse"].view(n_q, hq))

    rng = np.random.default_rng(7)
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
    # a one-window oracle call over the blocks that read it
    checked = 0
    for b in (0, 3, 7):
        gsb = P["plan_gs"][b].cpu().numpy()
        glb = P["plan_gl"][b].cpu().numpy()
        for l0, g0, rd in pick_windows(meta, gsb, glb, rng, 2, 24):
            rrows = token_rows(rd)
            sub_r = sub_blocks(meta, rd)
            ro_r, rl_r = oracle.sparse_xattn_fwd(q64[rrows], k64, v64, sub_r.anchor,
                                                 sub_r.sample_start, gs_all, gl_all, scale,
                                                 ks64[rrows], vs64[rrows])
            g1, l1 = np.array([g0], np.int32), np.array([64], np.int32)
            rr = oracle.sparse_xattn_bwd(q64[rrows], k64[g0:g0 + 64], v64[g0:g0 + 64], ro_r,
                                         do64[rrows], rl_r, sub_r.anchor, sub_r.sample_start,
                                         g1, l1, scale)
            got_k = host64(P["dk_loc"][b][l0:l0 + 64])
            got_v = host64(P["dv_loc"][b][l0:l0 + 64])
            assert rel_frob(got_k, rr[1]) <= 3e-2, (b, l0, g0)
            assert rel_frob(got_v, rr[2]) <= 3e-2, (b, l0, g0)
            checked += 1
    assert checked >= 4
