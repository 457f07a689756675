"""The split forward schedule (workspace "split"): row groups that read more key
tiles than 1.5 times a compute unit's mean share run as several pieces whose partial O and lse
a merge pass combines.

Checked against the oracle on whole outputs, against the unsplit call, and on the
plan itself.  P enters the output MFMAs in bf16 after subtracting the running row
maximum, and a piece keeps its own maximum, so P rounds differently than in the
unsplit walk: O agrees with the unsplit call to the bf16 rounding of P (relative
2^-9 per term), lse (float32 sums of unrounded P) to float32 rounding.  On the plan:
every split group's pieces cover its tile walk exactly once, in order, jobs are
dispatched longest piece first, and slots are distinct.  The tile count of a row group is restated here from its definition
(own-block tiles, then per chunk the 64-key tiles aligned to the chunk start that
meet [min sample start, max anchor) of the group's blocks).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth, sxattn
from helpers import assert_lse_close, dev, device_meta, host64, rel_frob

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROWS = 256


def group_tiles(meta, hq, hkv, gs, gl, with_self):
    grp = hq // hkv
    R = meta.n_blk * 16 * grp
    n_groups = -(-R // ROWS)
    out = np.zeros(n_groups, np.int64)
    for i in range(n_groups):
        r0, r1 = i * ROWS, min(i * ROWS + ROWS, R) - 1
        b0, b1 = r0 // grp // 16, r1 // grp // 16
        t = -(-16 * (b1 - b0 + 1) // 64) if with_self else 0
        lo = int(meta.sample_start[b0:b1 + 1].min())
        hi = int(meta.anchor[b0:b1 + 1].max())
        for s, n in zip(gs.tolist(), gl.tolist()):
            a, e = max(lo, s), min(hi, s + n)
            if a < e:
                t += -(-(e - s) // 64) - (a - s) // 64
        out[i] = t
    return out


def read_plan(n_groups, hkv):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    pieces = max(2, -(-2 * n_cu // hkv))
    ws = sxattn._workspaces[("fwd_split", torch.device("cuda", torch.cuda.current_device()),
                             torch.cuda.current_stream().cuda_stream)]
    jobs = ws[:16 * (n_groups + pieces)].cpu().numpy().view(np.int32).reshape(-1, 4)
    assert (jobs[:, 0] >= 0).sum() <= n_groups + max_extra(hkv)
    return jobs, pieces


def max_extra(hkv):
    """Spare job slots of the split grid per kv head: a group of T > cap tiles becomes
    ceil(T / cap) jobs and the tiles of all groups sum to at most cap 2 n_cu / (3 hkv)."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    return max(1, -(-2 * n_cu // (3 * hkv)))


def check_plan(jobs, pieces, tiles):
    n_groups = len(tiles)
    live = jobs[jobs[:, 0] >= 0]
    assert (jobs[len(live):, 0] == -1).all()          # live jobs first, then empty slots
    assert sorted(set(live[:, 0].tolist())) == list(range(n_groups))
    lengths = []
    slots = []
    for row in live:
        i, t0, t1, slot = (int(x) for x in row)
        if slot < 0:
            assert t0 == 0 and t1 == 0x7fffffff and (live[:, 0] == i).sum() == 1
            lengths.append(int(tiles[i]))
        else:
            slots.append(slot)
            lengths.append(t1 - t0)
    assert all(a >= b for a, b in zip(lengths, lengths[1:]))   # longest piece first
    assert len(set(slots)) == len(slots) and all(0 <= s < pieces for s in slots)
    n_split = 0
    for i in range(n_groups):
        mine = live[live[:, 0] == i]
        if (mine[:, 3] < 0).all():
            continue
        n_split += 1
        mine = mine[np.argsort(mine[:, 1])]
        assert mine[0, 1] == 0 and mine[-1, 2] == tiles[i]
        assert (mine[1:, 1] == mine[:-1, 2]).all() and (mine[:, 2] > mine[:, 1]).all()
        assert (np.diff(np.sort(mine[:, 3])) == 1).all()     # consecutive slots
    return n_split


CASES = [
    # (n_ctx, len_lo, len_hi, n_blk, hq, hkv, d, chunk list kind, with_self)
    (4096, 512, 2048, 32, 32, 8, 128, "contiguous", True),
    (16384, 1024, 16384, 64, 32, 8, 128, "ragged", True),
    (16384, 2048, 16384, 48, 8, 8, 128, "ragged", False),
    (12000, 300, 12000, 40, 40, 1, 64, "ragged", True),
    (8192, 8192, 8192, 20, 12, 4, 128, "contiguous", True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_split_forward_matches_oracle_and_unsplit(case, out_dtype):
    n_ctx, lo, hi, n_blk, hq, hkv, d, kind, with_self = CASES[case]
    seed = 40 + case
    meta = synth.draw_meta(seed, n_ctx, lo, hi, n_blk)
    if kind == "contiguous":
        gs, gl = synth.contiguous_chunks(n_ctx, 1024)
    else:   # ragged pieces listed out of order, some left out
        rng = np.random.default_rng(seed)
        cuts = np.sort(rng.choice(np.arange(1, n_ctx), 9, replace=False))
        starts = np.concatenate([[0], cuts]).astype(np.int32)
        lens = np.diff(np.concatenate([starts, [n_ctx]])).astype(np.int32)
        keep = rng.permutation(len(starts))[:8]
        gs, gl = starts[keep], lens[keep]
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "bf16", 1.0, gs, gl, self_block=with_self)
    scale = 1.0 / math.sqrt(d)
    dm = device_meta(meta, gs, gl)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    ks = dev(inp.k_self) if with_self else None
    vs = dev(inp.v_self) if with_self else None
    o_s, l_s = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, out_dtype=out_dtype,
                                       workspace="split")
    o_u, l_u = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, out_dtype=out_dtype,
                                       workspace=None)
    torch.cuda.synchronize()
    tiles = group_tiles(meta, hq, hkv, gs, gl, with_self)
    jobs, pieces = read_plan(len(tiles), hkv)
    n_split = check_plan(jobs, pieces, tiles)
    assert n_split > 0, "the case was meant to split some row group"

    ro, rl = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, gs, gl, scale,
                                     inp.k_self.f64 if with_self else None,
                                     inp.v_self.f64 if with_self else None)
    o = host64(o_s)
    assert np.abs(o - ro).max() <= 2e-2 and rel_frob(o, ro) <= 1e-2
    assert_lse_close(host64(l_s), rl, 1e-3)
    # against the unsplit call: the bf16 rounding of P (plus one of O for bf16 outputs)
    assert rel_frob(o, host64(o_u)) <= 4e-3
    assert_lse_close(host64(l_s), host64(l_u), 1e-5)


def test_split_workspace_reused_by_a_smaller_call_and_no_key_calls():
    """A second, smaller call rewrites the plan it shares; calls with only the
    own-block term, or with no key at all, behave as unsplit."""
    w = synth.WORKLOADS["fwd_bf16_512q_4k"]
    big = synth.draw_meta(7, 16384, 1024, 16384, 64)
    gs, gl = synth.contiguous_chunks(16384, 1024)
    inp = synth.draw_inputs(7, big, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl)
    sxattn.sparse_xattn_fwd(dev(inp.q), dev(inp.k), dev(inp.v), device_meta(big, gs, gl), 0.1,
                            dev(inp.k_self), dev(inp.v_self), workspace="split")
    small = synth.draw_meta(8, 4096, 512, 2048, 12)
    gs2, gl2 = np.array([2048, 0], np.int32), np.array([2048, 1024], np.int32)
    inp2 = synth.draw_inputs(8, small, w.hq, w.hkv, w.d, "bf16", 1.0, gs2, gl2)
    scale = 1.0 / math.sqrt(w.d)
    for cg, cl, with_self in ((gs2, gl2, True), (gs2[:0], gl2[:0], True), (gs2[:0], gl2[:0], False)):
        n_loc = int(cl.sum())
        dm = device_meta(small, cg, cl)
        k = dev(inp2.k)[:n_loc].contiguous() if n_loc else dev(inp2.k)[:0]
        v = dev(inp2.v)[:n_loc].contiguous() if n_loc else dev(inp2.v)[:0]
        ks = dev(inp2.k_self) if with_self else None
        vs = dev(inp2.v_self) if with_self else None
        o, lse = sxattn.sparse_xattn_fwd(dev(inp2.q), k, v, dm, scale, ks, vs,
                                         out_dtype=torch.float32, workspace="split")
        torch.cuda.synchronize()
        tiles = group_tiles(small, w.hq, w.hkv, cg, cl, with_self)
        jobs, pieces = read_plan(len(tiles), w.hkv)
        check_plan(jobs, pieces, tiles)
        ro, rl = oracle.sparse_xattn_fwd(inp2.q.f64, inp2.k.f64[:n_loc], inp2.v.f64[:n_loc],
                                         small.anchor, small.sample_start, cg, cl, scale,
                                         inp2.k_self.f64 if with_self else None,
                                         inp2.v_self.f64 if with_self else None)
        assert rel_frob(host64(o), ro) <= 1e-2 if ro.any() else not host64(o).any()
        assert_lse_close(host64(lse), rl, 1e-3)


def draw_case(case):
    n_ctx, lo, hi, n_blk, hq, hkv, d, kind, with_self = CASES[case]
    seed = 40 + case
    meta = synth.draw_meta(seed, n_ctx, lo, hi, n_blk)
    if kind == "contiguous":
        gs, gl = synth.contiguous_chunks(n_ctx, 1024)
    else:
        rng = np.random.default_rng(seed)
        cuts = np.sort(rng.choice(np.arange(1, n_ctx), 9, replace=False))
        starts = np.concatenate([[0], cuts]).astype(np.int32)
        lens = np.diff(np.concatenate([starts, [n_ctx]])).astype(np.int32)
        keep = rng.permutation(len(starts))[:8]
        gs, gl = starts[keep], lens[keep]
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "bf16", 1.0, gs, gl, self_block=with_self,
                            with_dout=True)
    return meta, inp, gs, gl, hq, hkv, d, with_self


@pytest.mark.parametrize("case", range(len(CASES)))
def test_split_dq_matches_unsplit_and_oracle(case):
    """The dQ phase on the split schedule: the same sums as the unsplit phase up to
    float32 summation order, accumulating into dq_accum or overwriting it; against the
    oracle (each side from its own forward) on the first two cases."""
    meta, inp, gs, gl, hq, hkv, d, with_self = draw_case(case)
    scale = 1.0 / math.sqrt(d)
    dm = device_meta(meta, gs, gl)
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    ks = dev(inp.k_self) if with_self else None
    vs = dev(inp.v_self) if with_self else None
    o, lse = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, workspace=None)
    delta = torch.empty((2,) + tuple(lse.shape), dtype=torch.float32, device="cuda")
    scratch_dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, scratch_dq, ks, vs, delta_ws=delta,
                            flags=sxattn.BWD_DELTA, workspace=None)
    init = torch.randn(q.shape, generator=torch.Generator().manual_seed(case)).cuda()
    out = {}
    for ws in ("auto", "split"):
        for mode, flags in (("acc", sxattn.BWD_DQ), ("over", sxattn.BWD_DQ | sxattn.BWD_DQ_OVERWRITE)):
            dq = init.clone()
            sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o, do, lse, dq, ks, vs, delta_ws=delta,
                                    flags=flags, workspace=ws)
            out[ws, mode] = dq
    torch.cuda.synchronize()
    # the split call left its plan at the start of the scratch's split region
    need = int(sxattn.load_library().sparse_xattn_bwd_workspace_bytes(meta.n_blk, int(gl.sum()), hq,
                                                                        hkv, d))
    base = -(-need // 256) * 256
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    pieces = max(2, -(-2 * n_cu // hkv))
    tiles = group_tiles(meta, hq, hkv, gs, gl, with_self)
    ws = sxattn._workspaces[("bwd_split", torch.device("cuda", torch.cuda.current_device()),
                             torch.cuda.current_stream().cuda_stream)]
    jobs = ws[base:base + 16 * (len(tiles) + pieces)].cpu().numpy().view(np.int32).reshape(-1, 4)
    assert (jobs[:, 0] >= 0).sum() <= len(tiles) + max_extra(hkv)
    assert check_plan(jobs, pieces, tiles) > 0
    dq_u = host64(out["auto", "over"])
    assert np.abs(dq_u).max() > 0
    assert rel_frob(host64(out["split", "over"]), dq_u) <= 1e-5
    assert rel_frob(host64(out["split", "acc"]) - host64(init), dq_u) <= 1e-5
    assert rel_frob(host64(out["split", "acc"]), host64(out["auto", "acc"])) <= 1e-6
    if case < 2:
        ks64 = inp.k_self.f64 if with_self else None
        vs64 = inp.v_self.f64 if with_self else None
        ro, rl = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                         meta.sample_start, gs, gl, scale, ks64, vs64)
        r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                    meta.anchor, meta.sample_start, gs, gl, scale, ks64, vs64)
        assert rel_frob(host64(out["split", "over"]), r[0]) <= 3e-2
