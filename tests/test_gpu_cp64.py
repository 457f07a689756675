"""One device's share at context-parallel size 64, checked against the oracle on
sampled outputs.

The full 8192-query view (512 blocks of 16) over a 524288-token packed context
(samples of 8192 to 65536 tokens), Hq 32, Hkv 8, d 128, bf16.  The GPU costs the 512
chunks of 1024 tokens, LPT plans them onto 64 bins, and bin 0's 8 non-contiguous
chunks are the local shard.  On it:
  * the partial forward (with the own-block term): O and lse of sampled blocks;
  * the 64-way combine of that partial with 63 synthetic partials, whose empty
    (block, bin) pattern is the real one (a partial is empty where the block's
    interval meets none of that bin's chunks);
  * the backward of the shard from the combined O and lse: dQ and the own-block
    dK, dV of sampled blocks, and dK, dV of 64-key windows of the shard: lightly read
    ones and the most heavily read ones (whose tiles the dK/dV schedule splits
    across workgroups).
A second test runs the mask-boundary probe (Q = 0, one-hot values; tests/probe.py)
on the shard and checks every output against its closed form.
The split schedule (forward and dQ) is compared with the default schedule on the
whole share.  The combine and the backward take the combined values only for the
blocks that are checked (sampled blocks and the readers of the windows; rows are independent),
and every other row keeps the shard's own partial.  The oracle's side is its own:
its forward of those blocks, its combine with the same synthetic partials, its
backward from that.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import probe
from block_sparse_cross_anchor_amd import synth, sxattn
from helpers import (assert_lse_close, dev, device_meta, dkdv_split_tiles, head_rows,
                     heavy_windows, host64, pick_windows, rel_frob, share_pairs, sub_blocks,
                     token_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_cp64_bin0_share_forward_combine_backward_sampled():
    w = synth.WORKLOADS["cp64_share_8kq_512k"]
    seed = 5
    n_q, hq, hkv, d, nb = w.n_q, w.hq, w.hkv, w.d, w.n_bin
    scale = 1.0 / math.sqrt(d)
    meta = synth.meta_for(w, seed)
    anchor = torch.as_tensor(meta.anchor).cuda()
    start = torch.as_tensor(meta.sample_start).cuda()
    cost = sxattn.chunk_cost(anchor, start, w.n_ctx, w.chunk_size).cpu()
    bins = sxattn.lpt_assign(cost, nb)[0].numpy()
    gs_all, gl_all = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    mine = np.flatnonzero(bins == 0)
    gs, gl = gs_all[mine], gl_all[mine]
    assert len(gs) == w.n_chunk // nb and np.any(np.diff(gs) != w.chunk_size)  # non-contiguous
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "bf16", w.std(), gs, gl, with_dout=True)
    q, k, v, ks, vs, do = (dev(t) for t in (inp.q, inp.k, inp.v, inp.k_self, inp.v_self, inp.dout))
    dm = device_meta(meta, gs, gl)

    # ---- partial forward of the shard; the split schedule on the whole share agrees
    # with it to the bf16 rounding of P
    o_p, l_p = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs)
    o_s, l_s = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, workspace="split")
    torch.cuda.synchronize()
    assert rel_frob(host64(o_s), host64(o_p)) <= 4e-3
    assert_lse_close(host64(l_s), host64(l_p), 1e-5)
    del o_s, l_s

    # blocks to check: first and last, blocks whose interval meets the shard, and the
    # readers of three 64-key windows of the shard
    lo = meta.sample_start.astype(np.int64)[:, None]
    hi = meta.anchor.astype(np.int64)[:, None]
    cs = gs_all.astype(np.int64)[None, :]
    meets_chunk = np.maximum(lo, cs) < np.minimum(hi, cs + gl_all[None, :])   # [n_blk, n_chunk]
    reach = np.flatnonzero(meets_chunk[:, mine].any(1))
    assert reach.size > 0
    rng = np.random.default_rng(11)
    sampled = np.unique(np.concatenate([[0, meta.n_blk - 1], rng.choice(reach, 6, replace=False),
                                        rng.integers(0, meta.n_blk, 2)]))
    windows = pick_windows(meta, gs, gl, rng, 3, 24)
    assert len(windows) == 3
    # and the most heavily read windows of the shard, whose tiles the dK/dV schedule
    # splits across workgroups and adds up in its fix-up pass
    heavy = heavy_windows(meta, gs, gl, 3, 2e7, pairs_of=lambda r: share_pairs(meta, r, gs, gl))
    assert len(heavy) >= 3 and heavy[0][2].size > 24
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    shares = dkdv_split_tiles(meta, gs, gl, hq, hkv, n_cu, True)
    assert sum(int(shares[l0 // 256] >= 2) for l0, _, _ in heavy) >= 1
    windows += heavy
    need = np.unique(np.concatenate([sampled] + [r for _, _, r in windows]))
    sub = sub_blocks(meta, need)
    trows = token_rows(need)
    hrows = head_rows(need, hq)
    pos = {int(b): i for i, b in enumerate(need)}   # block -> index in `need`

    q64, k64, v64, do64 = inp.q.f64[trows], inp.k.f64, inp.v.f64, inp.dout.f64[trows]
    ks64, vs64 = inp.k_self.f64[trows], inp.v_self.f64[trows]
    ro_p, rl_p = oracle.sparse_xattn_fwd(q64, k64, v64, sub.anchor, sub.sample_start, gs, gl,
                                         scale, ks64, vs64)
    sel = torch.as_tensor(trows).cuda()
    o_got = host64(o_p[sel])
    assert np.abs(o_got - ro_p).max() <= 2e-2 and rel_frob(o_got, ro_p) <= 1e-2
    assert_lse_close(host64(l_p[sel]), rl_p, 1e-3)

    # ---- 64-way combine on the rows of `need`
    meets_bin = np.stack([meets_chunk[:, bins == p].any(1) for p in range(nb)])  # [nb, n_blk]
    empty = ~meets_bin[1:, need]                                       # [63, len(need)]
    empty = np.repeat(empty, 16 * hq, axis=1)                          # -> head rows
    o_syn, l_syn = synth.draw_partials(seed, nb - 1, hrows.size, d, "bf16", empty=empty)
    hsel = torch.as_tensor(hrows).cuda()
    parts_o = torch.cat([o_p.view(-1, d)[hsel].unsqueeze(0), dev(o_syn)])
    parts_l = torch.cat([l_p.view(-1)[hsel].unsqueeze(0), torch.as_tensor(l_syn).cuda()])
    co, cl = sxattn.lse_combine(parts_o, parts_l)
    torch.cuda.synchronize()
    ro_f, rl_f = oracle.lse_combine(
        np.concatenate([ro_p.reshape(1, -1, d), o_syn.f64]),
        np.concatenate([rl_p.reshape(1, -1), l_syn.astype(np.float64)]))
    assert np.abs(host64(co) - ro_f).max() <= 2e-2 and rel_frob(host64(co), ro_f) <= 1e-2
    assert_lse_close(host64(cl), rl_f, 1e-3)

    # ---- backward of the shard from the combined O and lse
    o_in = o_p.clone().view(-1, d)
    l_in = l_p.clone().view(-1)
    o_in[hsel] = co
    l_in[hsel] = cl
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o_in.view(n_q, hq, d), do,
                                               l_in.view(n_q, hq), dq, ks, vs)
    dq_s = torch.zeros(q.shape, dtype=torch.float32, device="cuda")   # dQ on the split schedule
    sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o_in.view(n_q, hq, d), do, l_in.view(n_q, hq), dq_s,
                            ks, vs, flags=sxattn.BWD_DELTA | sxattn.BWD_DQ, workspace="split")
    torch.cuda.synchronize()
    assert rel_frob(host64(dq_s), host64(dq)) <= 1e-5
    del dq_s
    ro_f = ro_f.reshape(-1, hq, d)
    rl_f = rl_f.reshape(-1, hq)

    def rows_of(blocks):   # rows of `blocks` inside the arrays over `need`
        return np.concatenate([np.arange(16 * pos[int(b)], 16 * pos[int(b)] + 16) for b in blocks])

    sr = rows_of(sampled)
    sub_s = sub_blocks(meta, sampled)
    r = oracle.sparse_xattn_bwd(q64[sr], k64, v64, ro_f[sr], do64[sr], rl_f[sr], sub_s.anchor,
                                sub_s.sample_start, gs, gl, scale, ks64[sr], vs64[sr])
    srows = token_rows(sampled)
    assert rel_frob(host64(dq)[srows], r[0]) <= 3e-2
    assert rel_frob(host64(dks)[srows], r[3]) <= 3e-2
    assert rel_frob(host64(dvs)[srows], r[4]) <= 3e-2
    for l0, g0, rd in windows:
        wr = rows_of(rd)
        sub_r = sub_blocks(meta, rd)
        g1, l1 = np.array([g0], np.int32), np.array([64], np.int32)
        rr = oracle.sparse_xattn_bwd(q64[wr], k64[l0:l0 + 64], v64[l0:l0 + 64], ro_f[wr],
                                     do64[wr], rl_f[wr], sub_r.anchor, sub_r.sample_start,
                                     g1, l1, scale)
        assert np.abs(rr[1]).max() > 0
        assert rel_frob(host64(dk)[l0:l0 + 64], rr[1]) <= 3e-2, (l0, g0)
        assert rel_frob(host64(dv)[l0:l0 + 64], rr[2]) <= 3e-2, (l0, g0)


def test_cp64_bin0_share_boundary_probe_all_outputs():
    """Q = 0 with one-hot probe values on bin 0's shard (own-block term included),
    forward then backward from the shard's own O and lse: O and lse of all 262144 query
    rows, dV of all 8192 local keys (per 256-key tile), dK = 0, and dQ of every row,
    against the closed forms of tests/probe.py (pinned against the oracle on the CPU)."""
    w = synth.WORKLOADS["cp64_share_8kq_512k"]
    seed = 5
    n_q, hq, hkv, d, nb = w.n_q, w.hq, w.hkv, w.d, w.n_bin
    scale = 1.0 / math.sqrt(d)
    meta = synth.meta_for(w, seed)
    anchor = torch.as_tensor(meta.anchor).cuda()
    start = torch.as_tensor(meta.sample_start).cuda()
    cost = sxattn.chunk_cost(anchor, start, w.n_ctx, w.chunk_size).cpu()
    bins = sxattn.lpt_assign(cost, nb)[0].numpy()
    gs_all, gl_all = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    mine = np.flatnonzero(bins == 0)
    gs, gl = gs_all[mine], gl_all[mine]
    inp = probe.inputs(seed, meta, hq, hkv, d, gs, gl, w.chunk_size)
    q, k, v, ks, vs, do = (dev(t) for t in (inp.q, inp.k, inp.v, inp.k_self, inp.v_self, inp.dout))
    dm = device_meta(meta, gs, gl)
    o, lse = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq, ks, vs)
    torch.cuda.synchronize()
    n_b, hits = probe.forward(meta, gs, gl, w.chunk_size, seed)
    want = np.repeat(hits / n_b[:, None], 16, axis=0)[:, None, :]
    og = host64(o)
    err = np.abs(og[..., :probe.N_COLS] - want)
    assert np.all(err <= 2 ** -8 * want + 1e-6), float(err.max())
    assert np.all(og[..., probe.N_COLS:] == 0)
    np.testing.assert_allclose(host64(lse), np.repeat(np.log(n_b), 16)[:, None] * np.ones((1, hq)),
                               rtol=0, atol=1e-5)
    want_v = probe.dv_context(meta, inp, gs, gl, hq, hkv)
    got_v = host64(dv)
    for t0 in range(0, want_v.shape[0], 256):
        assert rel_frob(got_v[t0:t0 + 256], want_v[t0:t0 + 256]) <= 1e-2, t0
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dks).item() == 0
    assert rel_frob(host64(dvs), probe.dv_self(meta, inp, gs, gl, hq, hkv)) <= 1e-2
    want_q = probe.dq(meta, inp, gs, gl, hq, hkv, scale, w.chunk_size, seed)
    got_q = host64(dq)
    assert rel_frob(got_q, want_q) <= 1e-2
    for b in range(meta.n_blk):
        r = slice(16 * b, 16 * b + 16)
        assert rel_frob(got_q[r], want_q[r]) <= 3e-2, b
