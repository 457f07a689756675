"""Blocks in any order: forward, combine and backward against the oracle.

The C ABI takes the query blocks in any order (anchor and sample start per block,
query rows 16 b .. 16 b + 15); performance assumes the generator's order, sorted by
(sample start, anchor), but results may not depend on it.  Here the blocks of the
512-query x 4096-token workload (Hq 32, Hkv 8, d 128, bf16) are permuted at random
-- metadata, Q, own-block K/V and dO rows alike -- and the whole path runs on the
permuted problem: one forward call per chunk (the own-block term on one of them),
the LSE combine, then the backward per chunk from the merged O and lse with dQ
accumulated over the calls, on each schedule (index order, the ranked dispatch
order with the load-balanced dK/dV, and the split schedule).  The oracle evaluates
the same permuted inputs.  A second case permutes the blocks of the 4096-query x
32768-token workload (8 chunks of 4096) and checks sampled blocks and key windows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth, sxattn
from helpers import (assert_lse_close, dev, device_meta, host64, pick_windows, rel_frob,
                     sub_blocks, token_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _permuted(w, seed, perm_seed):
    """The workload's metadata and inputs with the blocks in a random order."""
    meta = synth.meta_for(w, seed)
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl,
                            with_dout=True)
    perm = np.random.default_rng(perm_seed).permutation(meta.n_blk)
    assert np.any(perm != np.arange(meta.n_blk))
    rows = token_rows(perm)
    meta_p = synth.Meta(meta.lengths, meta.offsets, meta.anchor[perm].copy(),
                        meta.sample_start[perm].copy(), meta.n_ctx)
    for name in ("q", "k_self", "v_self", "dout"):
        t = getattr(inp, name)
        setattr(inp, name, synth.Tensor(np.ascontiguousarray(t.bits[rows]), t.dtype))
    return meta_p, inp, gs, gl


def _gpu_path(meta, inp, gs, gl, scale, workspace):
    """Forward per chunk, combine, backward per chunk (dQ accumulated)."""
    q, ks, vs, do = dev(inp.q), dev(inp.k_self), dev(inp.v_self), dev(inp.dout)
    k_all, v_all = dev(inp.k), dev(inp.v)
    offs = np.concatenate([[0], np.cumsum(gl)])
    n_q, hq, d = q.shape
    self_chunk = len(gs) // 2          # the own-block term rides on a middle chunk
    parts_o, parts_l, calls = [], [], []
    for c in range(len(gs)):
        m = sxattn.Meta(meta.anchor, meta.sample_start, gs[c:c + 1], gl[c:c + 1])
        k = k_all[int(offs[c]):int(offs[c + 1])]
        v = v_all[int(offs[c]):int(offs[c + 1])]
        sk = (ks, vs) if c == self_chunk else (None, None)
        o_p, l_p = sxattn.sparse_xattn_fwd(q, k, v, m, scale, *sk, workspace=workspace)
        parts_o.append(o_p.view(-1, d))
        parts_l.append(l_p.view(-1))
        calls.append((m, k, v, sk))
    o, lse = sxattn.lse_combine(torch.stack(parts_o), torch.stack(parts_l))
    o, lse = o.view(n_q, hq, d), lse.view(n_q, hq)
    dq = torch.empty((n_q, hq, d), dtype=torch.float32, device="cuda")
    delta = torch.empty((2, n_q, hq), dtype=torch.float32, device="cuda")
    dk = torch.empty(k_all.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    dks = torch.empty(ks.shape, dtype=torch.float32, device="cuda")
    dvs = torch.empty_like(dks)
    for c, (m, k, v, sk) in enumerate(calls):
        flags = sxattn.BWD_DQ | sxattn.BWD_DKDV | (sxattn.BWD_DELTA | sxattn.BWD_DQ_OVERWRITE
                                                   if c == 0 else 0)
        sxattn.sparse_xattn_bwd(q, k, v, m, scale, o, do, lse, dq, *sk, delta_ws=delta,
                                dk=dk[int(offs[c]):int(offs[c + 1])],
                                dv=dv[int(offs[c]):int(offs[c + 1])], dk_self=dks, dv_self=dvs,
                                flags=flags, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv, dks, dvs


@pytest.mark.parametrize("seed,perm_seed", [(2, 40), (102, 41)])
@pytest.mark.parametrize("workspace", [None, "auto", "split"])
def test_permuted_blocks_small_whole_path(seed, perm_seed, workspace):
    w = synth.WORKLOADS["fwd_bf16_512q_4k"]
    meta, inp, gs, gl = _permuted(w, seed, perm_seed)
    scale = 1.0 / math.sqrt(w.d)
    o, lse, dq, dk, dv, dks, dvs = _gpu_path(meta, inp, gs, gl, scale, workspace)
    ro, rl = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, gs, gl, scale, inp.k_self.f64,
                                     inp.v_self.f64)
    og = host64(o)
    assert np.abs(og - ro).max() <= 2e-2 and rel_frob(og, ro) <= 1e-2
    assert_lse_close(host64(lse), rl, 1e-3)
    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale, inp.k_self.f64,
                                inp.v_self.f64)
    for got, want, name in ((dq, r[0], "dq"), (dk, r[1], "dk"), (dv, r[2], "dv"),
                            (dks, r[3], "dk_self"), (dvs, r[4], "dv_self")):
        err = rel_frob(host64(got), want)
        assert err <= 3e-2, f"{name}: relative Frobenius error {err:.3e}"


def test_permuted_blocks_4k_queries_32k_context_sampled():
    w = synth.WORKLOADS["fwdbwd_bf16_4kq_32k"]
    meta, inp, gs, gl = _permuted(w, 4, 42)
    scale = 1.0 / math.sqrt(w.d)
    o, lse, dq, dk, dv, dks, dvs = _gpu_path(meta, inp, gs, gl, scale, "auto")
    rng = np.random.default_rng(9)
    blocks = np.unique(np.concatenate([[0, meta.n_blk - 1], rng.integers(0, meta.n_blk, 6)]))
    windows = pick_windows(meta, gs, gl, rng, 4, 24)
    assert len(windows) >= 3
    need = np.unique(np.concatenate([blocks] + [r for _, _, r in windows]))
    sub = sub_blocks(meta, need)
    nrows = token_rows(need)
    q64, k64, v64, do64 = inp.q.f64[nrows], inp.k.f64, inp.v.f64, inp.dout.f64[nrows]
    ks64, vs64 = inp.k_self.f64[nrows], inp.v_self.f64[nrows]
    ro, rl = oracle.sparse_xattn_fwd(q64, k64, v64, sub.anchor, sub.sample_start, gs, gl, scale,
                                     ks64, vs64)
    og = host64(o)[nrows]
    assert np.abs(og - ro).max() <= 2e-2 and rel_frob(og, ro) <= 1e-2
    assert_lse_close(host64(lse)[nrows], rl, 1e-3)
    pos = {int(b): i for i, b in enumerate(need)}

    def rows_of(bl):
        return np.concatenate([np.arange(16 * pos[int(b)], 16 * pos[int(b)] + 16) for b in bl])

    sr = rows_of(blocks)
    sb = sub_blocks(meta, blocks)
    r = oracle.sparse_xattn_bwd(q64[sr], k64, v64, ro[sr], do64[sr], rl[sr], sb.anchor,
                                sb.sample_start, gs, gl, scale, ks64[sr], vs64[sr])
    trows = token_rows(blocks)
    assert rel_frob(host64(dq)[trows], r[0]) <= 3e-2
    assert rel_frob(host64(dks)[trows], r[3]) <= 3e-2
    assert rel_frob(host64(dvs)[trows], r[4]) <= 3e-2
    for l0, g0, rd in windows:
        wr = rows_of(rd)
        s_r = sub_blocks(meta, rd)
        rr = oracle.sparse_xattn_bwd(q64[wr], k64[l0:l0 + 64], v64[l0:l0 + 64], ro[wr], do64[wr],
                                     rl[wr], s_r.anchor, s_r.sample_start,
                                     np.array([g0], np.int32), np.array([64], np.int32), scale)
        assert rel_frob(host64(dk)[l0:l0 + 64], rr[1]) <= 3e-2, (l0, g0)
        assert rel_frob(host64(dv)[l0:l0 + 64], rr[2]) <= 3e-2, (l0, g0)
