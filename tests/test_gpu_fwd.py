"""GPU parity of the forward, combine, cost and LPT path against the CPU oracle.

Tolerances: cost and LPT bit-exact; float32 attention 1e-5 relative (Frobenius);
bf16 attention O max-abs 2e-2 and relative-Frobenius 1e-2, lse abs 1e-3 with -inf
rows matching exactly; combine of float32 partials 1e-5.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth, sxattn
from helpers import assert_lse_close, dev, device_meta, host64, rel_frob, sub_blocks, token_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

W = synth.WORKLOADS


def fwd_case(w, seed, gs, gl, self_block=True, std=None, dtype=None):
    meta = synth.meta_for(w, seed)
    std = w.std() if std is None else std
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, dtype or w.dtype, std, gs, gl,
                            self_block=self_block)
    return meta, inp


def run_fwd(meta, inp, scale, gs=None, gl=None, k=None, v=None, with_self=True, out_dtype=None):
    gs = inp.chunk_gstart if gs is None else gs
    gl = inp.chunk_len if gl is None else gl
    dm = device_meta(meta, gs, gl)
    kd = dev(inp.k) if k is None else k
    vd = dev(inp.v) if v is None else v
    o, lse = sxattn.sparse_xattn_fwd(dev(inp.q), kd, vd, dm, scale,
                                     dev(inp.k_self) if with_self else None,
                                     dev(inp.v_self) if with_self else None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


def oracle_fwd(meta, inp, scale, with_self=True, gs=None, gl=None, k=None, v=None):
    gs = inp.chunk_gstart if gs is None else gs
    gl = inp.chunk_len if gl is None else gl
    return oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64 if k is None else k,
                                   inp.v.f64 if v is None else v, meta.anchor, meta.sample_start,
                                   gs, gl, scale, inp.k_self.f64 if with_self else None,
                                   inp.v_self.f64 if with_self else None)


def check_bf16(o_gpu, lse_gpu, o_ref, lse_ref):
    o = host64(o_gpu)
    assert np.abs(o - o_ref).max() <= 2e-2
    assert rel_frob(o, o_ref) <= 1e-2
    assert_lse_close(host64(lse_gpu), lse_ref, 1e-3)


# ----------------------------------------------------------------------------- cost + LPT

@pytest.mark.parametrize("name", list(W))
def test_chunk_cost_bit_exact(name):
    w = W[name]
    meta = synth.meta_for(w, 1)
    a = torch.as_tensor(meta.anchor).cuda()
    s = torch.as_tensor(meta.sample_start).cuda()
    got = sxattn.chunk_cost(a, s, w.n_ctx, w.chunk_size).cpu().numpy()
    assert got.dtype == np.int64 and got.shape == (w.n_chunk,)
    assert int(got.sum()) == 16 * int((meta.anchor.astype(np.int64) - meta.sample_start).sum())
    idx = np.arange(w.n_chunk) if w.n_chunk <= 64 else \
        np.unique(np.random.default_rng(0).integers(0, w.n_chunk, 48))
    want = oracle.chunk_cost(meta.anchor, meta.sample_start, w.n_ctx, w.chunk_size, chunks=idx)
    np.testing.assert_array_equal(got[idx], want)


@pytest.mark.parametrize("seed", range(6))
def test_chunk_cost_ragged_and_edge_cases(seed):
    rng = np.random.default_rng(seed)
    n_ctx = int(rng.integers(50, 3000))
    meta = synth.draw_meta(seed, n_ctx, 40, 700, int(rng.integers(1, 20)))
    for cs in (1, 7, 64, int(rng.integers(1, n_ctx + 1)), n_ctx + 5):
        got = sxattn.chunk_cost(torch.as_tensor(meta.anchor).cuda(),
                                torch.as_tensor(meta.sample_start).cuda(), n_ctx, cs).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.chunk_cost(meta.anchor, meta.sample_start,
                                                             n_ctx, cs))
    # no blocks: all-zero costs; empty context: nothing to write
    z = sxattn.chunk_cost(torch.zeros(0, dtype=torch.int32, device="cuda"),
                          torch.zeros(0, dtype=torch.int32, device="cuda"), 100, 30)
    assert z.cpu().tolist() == [0, 0, 0, 0]
    e = sxattn.chunk_cost(torch.as_tensor(meta.anchor).cuda(),
                          torch.as_tensor(meta.sample_start).cuda(), 0, 30)
    assert e.numel() == 0


def test_chunk_cost_int64_range():
    n_blk = 40000
    a = torch.full((n_blk,), 4096, dtype=torch.int32, device="cuda")
    s = torch.zeros(n_blk, dtype=torch.int32, device="cuda")
    got = sxattn.chunk_cost(a, s, 4096, 4096).cpu().tolist()
    assert got == [16 * n_blk * 4096]


@pytest.mark.parametrize("name", ["fwd_bf16_8kq_64k", "cp64_share_8kq_512k"])
def test_gpu_cost_then_lpt_plan_matches_oracle(name):
    w = W[name]
    meta = synth.meta_for(w, 2)
    cost = sxattn.chunk_cost(torch.as_tensor(meta.anchor).cuda(),
                             torch.as_tensor(meta.sample_start).cuda(), w.n_ctx, w.chunk_size)
    bins, load = sxattn.lpt_assign(cost.cpu(), w.n_bin)
    want_bins, want_load = oracle.lpt_assign(cost.cpu().numpy(), w.n_bin)
    assert bins.tolist() == want_bins and load.tolist() == want_load
    assert oracle.imbalance(want_load) < 0.05


# ----------------------------------------------------------------------------- combine

@pytest.mark.parametrize("in_dt,out_dt", [("f32", torch.float32), ("bf16", torch.bfloat16),
                                          ("bf16", torch.float32)])
@pytest.mark.parametrize("n_parts,rows,d", [(1, 37, 128), (5, 1000, 128), (64, 333, 128),
                                            (3, 50, 64), (9, 17, 256)])
def test_lse_combine_matches_oracle(in_dt, out_dt, n_parts, rows, d):
    rng = np.random.default_rng(n_parts * 1000 + rows)
    empty = rng.random((n_parts, rows)) < 0.3
    empty[:, :3] = True  # rows whose partials are all empty
    o, lse = synth.draw_partials(rows + d, n_parts, rows, d, in_dt, empty=empty)
    lse_t = torch.as_tensor(lse).cuda()
    go, gl = sxattn.lse_combine(dev(o), lse_t, out_dtype=out_dt)
    torch.cuda.synchronize()
    want_o, want_l = oracle.lse_combine(o.f64, lse.astype(np.float64))
    assert_lse_close(host64(gl), want_l, 1e-5)
    got = host64(go)
    if out_dt == torch.float32 and in_dt == "f32":
        assert rel_frob(got, want_o) <= 1e-5
    else:
        assert np.abs(got - want_o).max() <= 2e-2 and rel_frob(got, want_o) <= 1e-2
    assert np.all(got[:3] == 0)


def test_lse_combine_skips_empty_partials_without_reading_them():
    rows, d = 64, 128
    o, lse = synth.draw_partials(5, 2, rows, d, "f32")
    lse[1, :] = -np.inf
    o.bits[1] = np.nan  # never read
    go, gl = sxattn.lse_combine(dev(o), torch.as_tensor(lse).cuda())
    torch.cuda.synchronize()
    np.testing.assert_allclose(host64(go), o.f64[0], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(host64(gl), lse[0], rtol=1e-6)


# ----------------------------------------------------------------------------- forward

def test_fwd_tiny_fp32_two_chunks_then_combine():
    """One 512-token sample, 4 anchors, hq = hkv = 2, d = 64, float32; two contiguous
    chunks; own-block term on the first call; partials merged on the GPU."""
    w = W["tiny_fp32_512"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta, inp = fwd_case(w, 1, gs, gl)
    scale = 1.0 / math.sqrt(w.d)
    parts_o, parts_l = [], []
    ref_o, ref_l = [], []
    offs = np.concatenate([[0], np.cumsum(gl)])
    for c in range(len(gs)):
        kd = dev(inp.k)[offs[c]:offs[c + 1]].contiguous()
        vd = dev(inp.v)[offs[c]:offs[c + 1]].contiguous()
        o, l = run_fwd(meta, inp, scale, gs[c:c + 1], gl[c:c + 1], kd, vd, with_self=(c == 0))
        ro, rl = oracle_fwd(meta, inp, scale, c == 0, gs[c:c + 1], gl[c:c + 1],
                            inp.k.f64[offs[c]:offs[c + 1]], inp.v.f64[offs[c]:offs[c + 1]])
        assert rel_frob(host64(o), ro) <= 1e-5
        assert_lse_close(host64(l), rl, 1e-5)
        parts_o.append(o)
        parts_l.append(l)
    co, cl = sxattn.lse_combine(torch.stack(parts_o).reshape(2, -1, w.d),
                                torch.stack(parts_l).reshape(2, -1))
    torch.cuda.synchronize()
    uo, ul = oracle_fwd(meta, inp, scale)
    assert rel_frob(host64(co), uo.reshape(-1, w.d)) <= 1e-5
    assert_lse_close(host64(cl), ul.reshape(-1), 1e-5)


@pytest.mark.parametrize("seed", [1, 101, 102])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fwd_bf16_4k_chunks_and_combine(seed, out_dtype):
    """4096-token context, 512 queries, GQA 32/8, d = 128, 4 chunks of 1024."""
    w = W["fwd_bf16_512q_4k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    meta, inp = fwd_case(w, seed, gs, gl)
    scale = 1.0 / math.sqrt(w.d)
    # unsplit call over all four chunks
    o, l = run_fwd(meta, inp, scale, out_dtype=out_dtype)
    uo, ul = oracle_fwd(meta, inp, scale)
    check_bf16(o, l, uo, ul)
    # one call per chunk, then the combine
    offs = np.concatenate([[0], np.cumsum(gl)])
    kd_all, vd_all = dev(inp.k), dev(inp.v)
    po, pl = [], []
    for c in range(len(gs)):
        sl = slice(offs[c], offs[c + 1])
        o_c, l_c = run_fwd(meta, inp, scale, gs[c:c + 1], gl[c:c + 1], kd_all[sl].contiguous(),
                           vd_all[sl].contiguous(), with_self=(c == 0), out_dtype=torch.float32)
        ro, rl = oracle_fwd(meta, inp, scale, c == 0, gs[c:c + 1], gl[c:c + 1], inp.k.f64[sl],
                            inp.v.f64[sl])
        check_bf16(o_c, l_c, ro, rl)
        po.append(o_c)
        pl.append(l_c)
    co, cl = sxattn.lse_combine(torch.stack(po).reshape(4, -1, w.d), torch.stack(pl).reshape(4, -1),
                                out_dtype=out_dtype)
    torch.cuda.synchronize()
    check_bf16(co, cl, uo.reshape(-1, w.d), ul.reshape(-1))


@pytest.mark.parametrize("seed", [3, 4])
def test_fwd_bf16_sharp_values_ragged_noncontiguous_chunks(seed):
    """Q, K, V ~ N(0, 1) (peaked softmax, so a wrong mask or scale shows), chunk
    lengths that are not multiples of the 64-key tile, chunks listed out of order
    and a subset of them (some rows have no allowed key)."""
    w = W["fwd_bf16_512q_4k"]
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, w.n_ctx), size=9, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int32)
    lens = np.diff(np.concatenate([starts, [w.n_ctx]])).astype(np.int32)
    keep = rng.permutation(len(starts))[:6]
    gs, gl = starts[keep], lens[keep]
    meta, inp = fwd_case(w, seed, gs, gl, std=1.0)
    scale = 1.0 / math.sqrt(w.d)
    for with_self in (True, False):
        o, l = run_fwd(meta, inp, scale, with_self=with_self, out_dtype=torch.float32)
        ro, rl = oracle_fwd(meta, inp, scale, with_self)
        check_bf16(o, l, ro, rl)
    # only the chunk that ends the context: blocks of earlier samples see no key
    gs1 = np.array([w.n_ctx - 1500], np.int32)
    gl1 = np.array([1500], np.int32)
    inp1 = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", 1.0, gs1, gl1)
    o, l = run_fwd(meta, inp1, scale, with_self=False, out_dtype=torch.float32)
    ro, rl = oracle_fwd(meta, inp1, scale, False)
    assert np.isneginf(rl).any() and np.isfinite(rl).any()
    check_bf16(o, l, ro, rl)


def test_fwd_bf16_boundary_probe():
    """Q = 0 makes attention uniform over the allowed keys; V channel 0 is 1 only at
    probe positions (sample starts, anchor - 1, anchors, chunk edges).  O[i, h, 0] is
    then (#probes allowed) / (#allowed) and lse = ln(#allowed): an off-by-one at any
    boundary moves O by ~1/n and lse by ~1/n."""
    w = W["fwd_bf16_512q_4k"]
    gs, gl = synth.contiguous_chunks(w.n_ctx, 640)  # chunk edges off the 64-key grid
    meta, inp = fwd_case(w, 5, gs, gl)
    gpos = synth.chunk_rows(gs, gl)
    probes = set(meta.sample_start.tolist()) | set((meta.anchor - 1).tolist()) | \
        set(meta.anchor.tolist()) | set(gs.tolist()) | set((gs + gl - 1).tolist())
    vbits = np.zeros(inp.v.bits.shape, np.uint16)
    one = synth.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    for r, j in enumerate(gpos):
        if int(j) in probes:
            vbits[r, :, 0] = one
    inp.v = synth.Tensor(vbits, "bf16")
    inp.q = synth.Tensor(np.zeros_like(inp.q.bits), "bf16")
    o, l = run_fwd(meta, inp, 0.1, with_self=False, out_dtype=torch.float32)
    o, l = host64(o), host64(l)
    for b in range(meta.n_blk):
        allowed = [j for j in range(int(meta.sample_start[b]), int(meta.anchor[b]))]
        hit = sum(1 for j in allowed if j in probes)
        rows = slice(16 * b, 16 * b + 16)
        np.testing.assert_allclose(o[rows, :, 0], hit / len(allowed), rtol=1e-5)
        np.testing.assert_allclose(l[rows], math.log(len(allowed)), atol=1e-5)
        assert np.all(o[rows, :, 1:] == 0)


def test_fwd_only_self_and_empty_calls():
    """n_chunk = 0 with the own-block term gives the own-block partial alone; a call
    with neither gives lse = -inf and O = 0 everywhere."""
    w = W["fwd_bf16_512q_4k"]
    gs = np.zeros(0, np.int32)
    meta, inp = fwd_case(w, 6, gs, gs)
    scale = 1.0 / math.sqrt(w.d)
    o, l = run_fwd(meta, inp, scale)
    ro, rl = oracle_fwd(meta, inp, scale)
    check_bf16(o, l, ro, rl)
    o2, l2 = run_fwd(meta, inp, scale, with_self=False)
    assert torch.all(o2 == 0) and torch.all(torch.isneginf(l2))


def test_fwd_tiny_bf16_d64_and_gqa_variants():
    """d = 64 and group sizes 1, 2, 3, 8, 40 (rows of a wave span several blocks, a
    block spans several waves, or a token's heads span several waves)."""
    for hq, hkv, d in [(4, 4, 64), (8, 4, 128), (16, 2, 128), (4, 2, 64), (6, 2, 128), (40, 1, 64)]:
        meta = synth.draw_meta(7, 3000, 300, 1200, 12)
        gs, gl = synth.contiguous_chunks(3000, 700)
        inp = synth.draw_inputs(7, meta, hq, hkv, d, "bf16", 1.0, gs, gl)
        scale = 1.0 / math.sqrt(d)
        o, l = run_fwd(meta, inp, scale, out_dtype=torch.float32)
        ro, rl = oracle_fwd(meta, inp, scale)
        check_bf16(o, l, ro, rl)


def test_fwd_headline_shape_sampled_rows():
    """8192 queries x 65536-token context, GQA 32/8, d = 128, one unsplit call (the
    shape the benchmark times); rows of sampled blocks are checked against the oracle,
    which evaluates each block independently."""
    w = W["fwd_bf16_8kq_64k"]
    gs, gl = np.array([0], np.int32), np.array([w.n_ctx], np.int32)
    meta, inp = fwd_case(w, 3, gs, gl)
    scale = 1.0 / math.sqrt(w.d)
    o, l = run_fwd(meta, inp, scale)
    rng = np.random.default_rng(0)
    starts = np.flatnonzero(np.diff(meta.sample_start) != 0) + 1  # first block of each sample
    blocks = np.unique(np.concatenate([[0, meta.n_blk - 1], starts, starts - 1,
                                       rng.integers(0, meta.n_blk, 6)]))
    sub = sub_blocks(meta, blocks)
    rows = token_rows(blocks)
    ro, rl = oracle.sparse_xattn_fwd(inp.q.f64[rows], inp.k.f64, inp.v.f64, sub.anchor,
                                     sub.sample_start, gs, gl, scale, inp.k_self.f64[rows],
                                     inp.v_self.f64[rows])
    check_bf16(o[torch.as_tensor(rows).cuda()], l[torch.as_tensor(rows).cuda()], ro, rl)


# ----------------------------------------------------------------------------- redistribution

@pytest.mark.parametrize("row_shape,dtype", [((8, 128), torch.bfloat16), ((2, 64), torch.float32),
                                             ((1, 8), torch.bfloat16)])
def test_context_gather_bit_exact(row_shape, dtype):
    rng = np.random.default_rng(3)
    n = 5000
    src = torch.randn((n,) + row_shape, generator=torch.Generator().manual_seed(1)).to(dtype).cuda()
    cuts = np.sort(rng.choice(np.arange(1, n), size=11, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int32)
    lens = np.diff(np.concatenate([starts, [n]])).astype(np.int32)
    pick = rng.permutation(len(starts))[:7]
    gs, gl = starts[pick], lens[pick]
    out = sxattn.context_gather(src, torch.as_tensor(gs).cuda(), torch.as_tensor(gl).cuda(),
                                int(gl.sum()))
    torch.cuda.synchronize()
    want = src.cpu()[torch.as_tensor(synth.chunk_rows(gs, gl))]
    assert torch.equal(out.cpu(), want)


def test_fwd_and_dq_dispatch_order_does_not_change_results():
    """With a workspace the row groups are dispatched most-tiles-first; every row
    group is still computed by one workgroup, so O, lse and the dQ accumulation are
    bitwise identical to index-order dispatch."""
    w = W["fwd_bf16_8kq_64k"]
    gs, gl = np.array([0, 20480, 40960], np.int32), np.array([4096, 8192, 6144], np.int32)
    meta, inp = fwd_case(w, 5, gs, gl)
    blocks = np.arange(0, meta.n_blk, 5)[:96]  # 24 row groups of unequal cost
    meta_sub = sub_blocks(meta, blocks)
    rows = torch.from_numpy(token_rows(blocks)).cuda()
    q = dev(inp.q)[rows].contiguous()
    ks, vs = dev(inp.k_self)[rows].contiguous(), dev(inp.v_self)[rows].contiguous()
    dm = device_meta(meta_sub, gs, gl)
    scale = 1.0 / math.sqrt(w.d)
    k, v = dev(inp.k), dev(inp.v)
    o1, l1 = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, workspace=None)
    o2, l2 = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    do = torch.randn(o1.shape, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).cuda()
    delta = torch.empty((2,) + tuple(l1.shape), dtype=torch.float32, device="cuda")
    dqs = []
    for ws in (None, "auto"):
        dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
        sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o1, do, l1, dq, ks, vs, delta_ws=delta,
                                flags=sxattn.BWD_DELTA | sxattn.BWD_DQ, workspace=ws)
        dqs.append(dq)
    torch.cuda.synchronize()
    assert torch.equal(dqs[0], dqs[1])
    assert dqs[0].abs().max() > 0
