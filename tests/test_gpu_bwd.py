"""GPU parity of the backward path against the CPU oracle.

The backward takes the merged output O and log-sum-exp as inputs.  Each side runs
end to end: the GPU backward consumes the GPU forward's O and lse, the oracle
backward the oracle forward's, so no oracle input comes from the GPU path.  The two
differ by O's rounding to the input dtype and ~1e-4 in lse, far inside the gradient
bounds.  Tolerances: bf16 gradients relative Frobenius <= 3e-2; float32 gradients
1e-5.  At the 4096-query x 32768-context shape the oracle evaluates sampled blocks
(for dQ) and sampled 64-key windows (for dK/dV); an entry of either depends only on
the inputs, dO and the merged O and lse of the blocks involved, so the oracle's
forward runs for just those blocks.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth, sxattn
from helpers import dev, device_meta, host64, pick_windows, rel_frob, sub_blocks, token_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

W = synth.WORKLOADS


def gpu_fwd_merged(meta, inp, scale, dm):
    """Unsplit GPU forward: the merged O (in_dtype) and lse that the backward consumes."""
    o, lse = sxattn.sparse_xattn_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale,
                                     dev(inp.k_self), dev(inp.v_self))
    torch.cuda.synchronize()
    return o, lse


def oracle_merged(meta, inp, scale, gs, gl, blocks=None, with_self=True):
    """The oracle's merged forward over the chunks (O, lse) for `blocks` (all blocks
    when None): what the oracle backward consumes."""
    sub = meta if blocks is None else sub_blocks(meta, blocks)
    rows = slice(None) if blocks is None else token_rows(blocks)
    return oracle.sparse_xattn_fwd(inp.q.f64[rows], inp.k.f64, inp.v.f64, sub.anchor,
                                   sub.sample_start, gs, gl, scale,
                                   inp.k_self.f64[rows] if with_self else None,
                                   inp.v_self.f64[rows] if with_self else None)


def run_case(meta, inp, scale, gs, gl, tol, dq_init=None, workspace="auto"):
    dm = device_meta(meta, gs, gl)
    o, lse = gpu_fwd_merged(meta, inp, scale, dm)
    dq = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda") if dq_init is None \
        else dq_init.clone()
    dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale, o,
                                               dev(inp.dout), lse, dq, dev(inp.k_self),
                                               dev(inp.v_self), workspace=workspace)
    torch.cuda.synchronize()
    ro, rl = oracle_merged(meta, inp, scale, gs, gl)
    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale,
                                inp.k_self.f64, inp.v_self.f64)
    want_dq = r[0] if dq_init is None else r[0] + host64(dq_init)
    for got, want, name in ((dq, want_dq, "dq"), (dk, r[1], "dk"), (dv, r[2], "dv"),
                            (dks, r[3], "dk_self"), (dvs, r[4], "dv_self")):
        err = rel_frob(host64(got), want)
        assert err <= tol, f"{name}: relative Frobenius error {err:.3e} > {tol}"
    return o, lse


@pytest.mark.parametrize("seed", [1, 101])
def test_bwd_bf16_4k_unsplit(seed):
    w = W["fwd_bf16_512q_4k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta = synth.meta_for(w, seed)
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl,
                            with_dout=True)
    run_case(meta, inp, 1.0 / math.sqrt(w.d), gs, gl, 3e-2)


@pytest.mark.parametrize("seed", [2, 3])
def test_bwd_bf16_sharp_ragged_chunks_and_dq_accumulation(seed):
    """N(0,1) values, chunk edges off the tile grid, chunks out of order, and dq_accum
    holding earlier contributions (the call adds to it)."""
    w = W["fwd_bf16_512q_4k"]
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, w.n_ctx), size=7, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int32)
    lens = np.diff(np.concatenate([starts, [w.n_ctx]])).astype(np.int32)
    perm = rng.permutation(len(starts))
    gs, gl = starts[perm], lens[perm]
    meta = synth.meta_for(w, seed)
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", 1.0, gs, gl, with_dout=True)
    dq0 = torch.randn(inp.q.shape, dtype=torch.float32, device="cuda",
                      generator=torch.Generator(device="cuda").manual_seed(seed))
    run_case(meta, inp, 1.0 / math.sqrt(w.d), gs, gl, 3e-2, dq_init=dq0)


def test_bwd_bf16_gqa_and_head_dim_variants():
    """Group sizes 1, 2, 8 divide the 32-row query step; 3 does not (steps of 10
    tokens with 2 padding rows); 40 exceeds it (a token's heads span two steps)."""
    for hq, hkv, d in [(4, 4, 64), (8, 4, 128), (16, 2, 128), (4, 2, 64), (6, 2, 128), (3, 1, 64),
                       (40, 1, 64)]:
        meta = synth.draw_meta(8, 3000, 300, 1200, 12)
        gs, gl = synth.contiguous_chunks(3000, 700)
        inp = synth.draw_inputs(8, meta, hq, hkv, d, "bf16", 1.0, gs, gl, with_dout=True)
        for ws in ("auto", None):  # load-balanced dK/dV, and one workgroup per key tile
            run_case(meta, inp, 1.0 / math.sqrt(d), gs, gl, 3e-2, workspace=ws)


def test_bwd_fp32_tiny():
    w = W["tiny_fp32_512"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta = synth.meta_for(w, 4)
    inp = synth.draw_inputs(4, meta, w.hq, w.hkv, w.d, "f32", 1.0, gs, gl, with_dout=True)
    run_case(meta, inp, 1.0 / math.sqrt(w.d), gs, gl, 1e-5)


def test_bwd_per_chunk_calls_sum_to_unsplit():
    """One call per chunk (own-block term on the first), dq accumulated across calls,
    equals the oracle's unsplit backward."""
    w = W["fwd_bf16_512q_4k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta = synth.meta_for(w, 9)
    inp = synth.draw_inputs(9, meta, w.hq, w.hkv, w.d, "bf16", 1.0, gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = gpu_fwd_merged(meta, inp, scale, device_meta(meta, gs, gl))
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    offs = np.concatenate([[0], np.cumsum(gl)])
    dks = []
    for c in range(len(gs)):
        dm = device_meta(meta, gs[c:c + 1], gl[c:c + 1])
        sl = slice(int(offs[c]), int(offs[c + 1]))
        dk, dv, dk_s, dv_s = sxattn.sparse_xattn_bwd(
            q, k[sl].contiguous(), v[sl].contiguous(), dm, scale, o, do, lse, dq,
            dev(inp.k_self) if c == 0 else None, dev(inp.v_self) if c == 0 else None)
        dks.append((dk, dv, dk_s, dv_s))
    torch.cuda.synchronize()
    ro, rl = oracle_merged(meta, inp, scale, gs, gl)
    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale,
                                inp.k_self.f64, inp.v_self.f64)
    assert rel_frob(host64(dq), r[0]) <= 3e-2
    dk_all = np.concatenate([host64(x[0]) for x in dks])
    dv_all = np.concatenate([host64(x[1]) for x in dks])
    assert rel_frob(dk_all, r[1]) <= 3e-2
    assert rel_frob(dv_all, r[2]) <= 3e-2
    assert rel_frob(host64(dks[0][2]), r[3]) <= 3e-2
    assert rel_frob(host64(dks[0][3]), r[4]) <= 3e-2


def test_bwd_no_queries_zero_gradients():
    k = torch.randn(100, 2, 128, device="cuda").to(torch.bfloat16)
    dm = sxattn.Meta(np.zeros(0, np.int32), np.zeros(0, np.int32), [0], [100])
    q = torch.zeros(0, 4, 128, device="cuda", dtype=torch.bfloat16)
    dq = torch.zeros(0, 4, 128, device="cuda")
    lse = torch.zeros(0, 4, device="cuda")
    dk, dv, _, _ = sxattn.sparse_xattn_bwd(q, k, k, dm, 0.1, q, q, lse, dq,
                                           dk=torch.full(k.shape, 3.0, device="cuda"),
                                           dv=torch.full(k.shape, 3.0, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_4k_queries_32k_context_per_chunk_sampled():
    """4096 queries x 32768 context, GQA 32/8, d = 128, 8 chunks of 4096 with one
    backward call each (the layout of one device's chunks); dq accumulated over the
    calls.  Sampled blocks (dq) and sampled key rows (dk, dv) against the oracle."""
    w = W["fwdbwd_bf16_4kq_32k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta = synth.meta_for(w, 4)
    inp = synth.draw_inputs(4, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = gpu_fwd_merged(meta, inp, scale, device_meta(meta, gs, gl))
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    offs = np.concatenate([[0], np.cumsum(gl)])
    dks = dvs = None
    for c in range(len(gs)):
        dm = device_meta(meta, gs[c:c + 1], gl[c:c + 1])
        sl = slice(int(offs[c]), int(offs[c + 1]))
        dk_c, dv_c, dks_c, dvs_c = sxattn.sparse_xattn_bwd(
            q, k[sl].contiguous(), v[sl].contiguous(), dm, scale, o, do, lse, dq,
            dev(inp.k_self) if c == 0 else None, dev(inp.v_self) if c == 0 else None)
        dk[sl] = dk_c
        dv[sl] = dv_c
        if c == 0:
            dks, dvs = dks_c, dvs_c
    torch.cuda.synchronize()
    # dq of sampled blocks: every allowed key of those blocks over all chunks
    rng = np.random.default_rng(1)
    blocks = np.unique(np.concatenate([[0, meta.n_blk - 1], rng.integers(0, meta.n_blk, 6)]))
    sub = sub_blocks(meta, blocks)
    rows = token_rows(blocks)
    ro, rl = oracle_merged(meta, inp, scale, gs, gl, blocks)
    r = oracle.sparse_xattn_bwd(inp.q.f64[rows], inp.k.f64, inp.v.f64, ro,
                                inp.dout.f64[rows], rl, sub.anchor, sub.sample_start,
                                gs, gl, scale, inp.k_self.f64[rows], inp.v_self.f64[rows])
    assert rel_frob(host64(dq)[rows], r[0]) <= 3e-2
    assert rel_frob(host64(dks)[rows], r[3]) <= 3e-2
    assert rel_frob(host64(dvs)[rows], r[4]) <= 3e-2
    # dk, dv of sampled 64-key windows: a one-chunk oracle call over the blocks that
    # read the window, with those blocks' merged O and lse
    windows = pick_windows(meta, gs, gl, rng, 3, 24)
    assert len(windows) == 3
    for l0, g0, rd in windows:
        rrows = token_rows(rd)
        sub_r = sub_blocks(meta, rd)
        ro_r, rl_r = oracle_merged(meta, inp, scale, gs, gl, rd)
        g1, l1 = np.array([g0], np.int32), np.array([64], np.int32)
        rr = oracle.sparse_xattn_bwd(inp.q.f64[rrows], inp.k.f64[l0:l0 + 64],
                                     inp.v.f64[l0:l0 + 64], ro_r, inp.dout.f64[rrows], rl_r,
                                     sub_r.anchor, sub_r.sample_start, g1, l1, scale)
        assert np.abs(rr[1]).max() > 0
        assert rel_frob(host64(dk)[l0:l0 + 64], rr[1]) <= 3e-2, (l0, g0)
        assert rel_frob(host64(dv)[l0:l0 + 64], rr[2]) <= 3e-2, (l0, g0)


def test_bwd_phase_flags_match_one_call():
    """DELTA, DQ (overwrite), DKDV issued as separate calls give the same bits as
    one call with all phases on a zeroed dq_accum."""
    w = W["fwd_bf16_512q_4k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta = synth.meta_for(w, 12)
    inp = synth.draw_inputs(12, meta, w.hq, w.hkv, w.d, "bf16", 1.0, gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(w.d)
    dm = device_meta(meta, gs, gl)
    o, lse = gpu_fwd_merged(meta, inp, scale, dm)
    q, k, v, do, ks, vs = (dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.k_self),
                           dev(inp.v_self))
    dq1 = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    r1 = sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq1, ks, vs)
    dq2 = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")  # overwritten
    delta = torch.empty((2,) + tuple(lse.shape), dtype=torch.float32, device="cuda")
    sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq2, ks, vs, delta_ws=delta,
                            flags=sxattn.BWD_DELTA)
    sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq2, ks, vs, delta_ws=delta,
                            flags=sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE)
    r2 = sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq2, ks, vs, delta_ws=delta,
                                 flags=sxattn.BWD_DKDV)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    # dK/dV of tiles split between workgroups are sums of partials: equal up to order
    for a, b in zip(r1, r2):
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-6)
    # overwrite on a call whose chunks reach no query row clears dq_accum
    late = np.array([w.n_ctx - 1], np.int32), np.array([1], np.int32)
    dm1 = device_meta(meta, *late)
    dq3 = torch.full(q.shape, 7.0, dtype=torch.float32, device="cuda")
    sxattn.sparse_xattn_bwd(q, k[-1:].contiguous(), v[-1:].contiguous(), dm1, scale, o, do, lse,
                            dq3, delta_ws=delta, flags=sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE)
    torch.cuda.synchronize()
    ro, rl = oracle_merged(meta, inp, scale, gs, gl)
    want = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64[-1:], inp.v.f64[-1:], ro,
                                   inp.dout.f64, rl, meta.anchor, meta.sample_start,
                                   *late, scale)[0]
    np.testing.assert_allclose(host64(dq3), want, atol=1e-6)


def test_bwd_split_key_tiles_match_unsplit():
    """With the workspace, heavily read key tiles are split over several workgroups
    and their partial dK/dV summed by a second pass; without it each tile is one
    workgroup.  Both agree (up to float32 summation order) and match the oracle."""
    w = W["fwdbwd_bf16_4kq_32k"]
    gs, gl = np.array([0], np.int32), np.array([8192], np.int32)  # one 8192-key chunk
    meta = synth.meta_for(w, 6)
    inp = synth.draw_inputs(6, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(w.d)
    dm = device_meta(meta, gs, gl)
    o, lse = gpu_fwd_merged(meta, inp, scale, dm)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dm, scale, o, dev(inp.dout), lse)
    dq = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
    r_split = sxattn.sparse_xattn_bwd(*args, dq, flags=sxattn.BWD_DELTA | sxattn.BWD_DKDV)
    r_one = sxattn.sparse_xattn_bwd(*args, dq, flags=sxattn.BWD_DELTA | sxattn.BWD_DKDV,
                                    workspace=None)
    torch.cuda.synchronize()
    for a, b in zip(r_split[:2], r_one[:2]):
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-6)
    rows = np.arange(0, 256)  # the first key tile: read by every block of the first sample
    rd = np.flatnonzero((meta.sample_start < 256) & (meta.anchor > 0))
    assert rd.size > 8
    ro, rl = oracle_merged(meta, inp, scale, gs, gl, rd)
    sub = sub_blocks(meta, rd)
    qr = token_rows(rd)
    r = oracle.sparse_xattn_bwd(inp.q.f64[qr], inp.k.f64[rows], inp.v.f64[rows], ro,
                                inp.dout.f64[qr], rl, sub.anchor, sub.sample_start,
                                np.array([0], np.int32), np.array([256], np.int32), scale)
    assert np.abs(r[1]).max() > 0
    assert rel_frob(host64(r_split[0])[rows], r[1]) <= 3e-2
    assert rel_frob(host64(r_split[1])[rows], r[2]) <= 3e-2


@pytest.mark.parametrize("workspace", [None, "auto"])
def test_bwd_bf16_key_value_gradients(workspace):
    """SXA_BWD_DKDV_BF16: the key/value gradients (context and own-block) written as
    bf16 are the round-to-nearest-even of the float32 results of the same schedule
    (the sums are formed in float32 either way), and within the gradient bound of the
    oracle; on both the per-tile and the load-balanced (stream-K) dK/dV schedules, on
    ragged non-contiguous chunks."""
    w = W["fwd_bf16_512q_4k"]
    seed = 13
    meta = synth.meta_for(w, seed)
    gs = np.array([3072, 0, 1024], np.int32)
    gl = np.array([1000, 1024, 1024], np.int32)
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(w.d)
    dm = device_meta(meta, gs, gl)
    o, lse = gpu_fwd_merged(meta, inp, scale, dm)
    args = (dev(inp.q), dev(inp.k), dev(inp.v), dm, scale, o, dev(inp.dout), lse)
    ks, vs = dev(inp.k_self), dev(inp.v_self)
    dq32 = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
    g32 = sxattn.sparse_xattn_bwd(*args, dq32, ks, vs, workspace=workspace)
    dq16 = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
    g16 = sxattn.sparse_xattn_bwd(*args, dq16, ks, vs, workspace=workspace,
                                  grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dq16, dq32)
    ro, rl = oracle_merged(meta, inp, scale, gs, gl)
    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale,
                                inp.k_self.f64, inp.v_self.f64)
    for a, b, want, name in zip(g16, g32, r[1:], ("dk", "dv", "dk_self", "dv_self")):
        assert a.dtype == torch.bfloat16 and b.dtype == torch.float32
        assert torch.equal(a, b.to(torch.bfloat16)), name
        assert rel_frob(host64(a), want) <= 3e-2, name
    # no queries: bf16 zeros
    k = torch.randn(100, 2, 128, device="cuda").to(torch.bfloat16)
    m0 = sxattn.Meta(np.zeros(0, np.int32), np.zeros(0, np.int32), [0], [100])
    q0 = torch.zeros(0, 4, 128, device="cuda", dtype=torch.bfloat16)
    dk, dv, _, _ = sxattn.sparse_xattn_bwd(q0, k, k, m0, 0.1, q0, q0,
                                           torch.zeros(0, 4, device="cuda"),
                                           torch.zeros(0, 4, 128, device="cuda"),
                                           dk=torch.full(k.shape, 3.0, device="cuda").to(torch.bfloat16),
                                           dv=torch.full(k.shape, 3.0, device="cuda").to(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)



def longest_stream_k_segment(meta, n_blk, grp, n_ctx, n_shares, setup=10):
    """Hits of the longest segment the load-balanced dK/dV phase gives one share, for a
    single sample starting at token 0 and one kv head: per 256-key tile the query
    steps (32 rows from a token boundary) whose blocks read past the tile's first
    key, each hit tile also carrying `setup` list units, the list cut into n_shares
    equal parts."""
    ts = 32 // min(grp, 32)
    hcs = -(-grp // 32)
    n_q = 16 * n_blk
    t0 = np.arange(-(-n_q // ts)) * ts
    last = np.minimum(t0 + ts, n_q) - 1
    reach = np.repeat(np.maximum(meta.anchor[t0 // 16], meta.anchor[last // 16]).astype(np.int64), hcs)
    hits = (reach[None, :] > 256 * np.arange(n_ctx // 256)[:, None]).sum(1)
    units = (hits + setup) * (hits > 0)
    pre = np.concatenate([[0], np.cumsum(units)])
    j = np.arange(n_shares)
    a, e = j * pre[-1] // n_shares, (j + 1) * pre[-1] // n_shares
    seg = np.minimum(e[:, None], pre[1:][None]) - np.maximum(a[:, None], pre[:-1][None] + setup)
    return int(np.where(hits[None] > 0, seg, 0).max())


@pytest.mark.parametrize("hq,n_blk", [(40, 160), (8, 1536)])
def test_dkdv_stream_k_segments_longer_than_one_step_batch(hq, n_blk):
    """Stream-K segments of more than 1024 hit steps: a segment loads its first 1024
    steps from the count pass's list and collects the rest by scanning from the last
    listed step.  One 32768-token sample read by every block, one kv head (so the
    shares are long), a head group beyond the 32-row step (40) and within it (8): the
    load-balanced dK/dV phase must give the sums of the one-workgroup-per-tile phase
    (which only scans), to float32 summation order."""
    hkv, d, n_ctx = 1, 64, 32768
    meta = synth.draw_meta(31 + hq, n_ctx, n_ctx, n_ctx, n_blk)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert longest_stream_k_segment(meta, n_blk, hq // hkv, n_ctx, n_cu) > 1024
    gs, gl = synth.contiguous_chunks(n_ctx, 1024)
    inp = synth.draw_inputs(31 + hq, meta, hq, hkv, d, "bf16", 1.0 / math.sqrt(d), gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(d)
    dm = device_meta(meta, gs, gl)
    o, lse = sxattn.sparse_xattn_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale,
                                     dev(inp.k_self), dev(inp.v_self))
    out = {}
    for ws in ("auto", None):
        dq = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
        dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale, o,
                                                   dev(inp.dout), lse, dq, dev(inp.k_self),
                                                   dev(inp.v_self), workspace=ws)
        out[ws] = [host64(t) for t in (dk, dv, dks, dvs)]
    torch.cuda.synchronize()
    for got, want, name in zip(out["auto"], out[None], ("dk", "dv", "dk_self", "dv_self")):
        assert np.abs(want).max() > 0
        err = rel_frob(got, want)
        assert err <= 1e-5, f"{name}: relative Frobenius difference {err:.3e}"


def test_dkdv_stream_k_without_hit_lists():
    """Calls whose (tile, query step) lists would exceed 2^24 entries keep no lists:
    every stream-K segment then collects its steps by scanning.  A 256k-token context
    of 2048-token samples, 8192 queries, head group 40 (16384 query steps): the
    load-balanced dK/dV phase must give the one-workgroup-per-tile phase's sums."""
    hq, hkv, d, n_ctx, n_blk = 40, 1, 64, 1 << 18, 512
    n_tiles = n_ctx // 256 + 16 * n_blk // 256
    n_steps = 16 * n_blk * 2              # one token per step, two steps per token
    assert n_tiles * n_steps > 1 << 24
    meta = synth.draw_meta(77, n_ctx, 2048, 2048, n_blk)
    gs, gl = synth.contiguous_chunks(n_ctx, 1024)
    inp = synth.draw_inputs(77, meta, hq, hkv, d, "bf16", 1.0 / math.sqrt(d), gs, gl, with_dout=True)
    scale = 1.0 / math.sqrt(d)
    dm = device_meta(meta, gs, gl)
    o, lse = sxattn.sparse_xattn_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale,
                                     dev(inp.k_self), dev(inp.v_self))
    out = {}
    for ws in ("auto", None):
        dq = torch.zeros(inp.q.shape, dtype=torch.float32, device="cuda")
        dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(dev(inp.q), dev(inp.k), dev(inp.v), dm, scale, o,
                                                   dev(inp.dout), lse, dq, dev(inp.k_self),
                                                   dev(inp.v_self), workspace=ws)
        out[ws] = [host64(t) for t in (dk, dv, dks, dvs)]
    torch.cuda.synchronize()
    for got, want, name in zip(out["auto"], out[None], ("dk", "dv", "dk_self", "dv_self")):
        assert np.abs(want).max() > 0
        err = rel_frob(got, want)
        assert err <= 1e-5, f"{name}: relative Frobenius difference {err:.3e}"
