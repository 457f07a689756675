"""Randomised GPU parity sweep over small problems.

Each seeded case draws the number of blocks, the packed context (sample lengths and
anchors), the head layout (Hq, Hkv), the head dimension, the dtype and a chunk list:
a random subset of a random partition of the context (ragged lengths, chunks of one
token, chunks listed out of order), with or without the own-block term and with or
without the load-balancing workspaces (also with the split schedule of the forward
and dQ phases).  Values are N(0, 1), so the softmax is peaked
and a wrong mask or scale shows.  The forward, the split-then-combine of one call per
chunk, and the backward (each side end to end: GPU forward then GPU backward, oracle
forward then oracle backward) are compared with the oracle at the usual tolerances.
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

HEADS = [(1, 1), (2, 1), (4, 4), (8, 2), (6, 2), (12, 4), (32, 8), (40, 1)]


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    n_ctx = int(rng.integers(40, 5000))
    n_blk = int(rng.integers(1, 41))
    lo = int(rng.integers(33, 400))
    meta = synth.draw_meta(seed, n_ctx, lo, int(rng.integers(lo, 3000)), n_blk)
    hq, hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    d = int(rng.choice([64, 128]))
    dtype = "f32" if seed % 6 == 5 else "bf16"
    n_cut = int(rng.integers(0, min(12, n_ctx - 1) + 1))
    cuts = np.sort(rng.choice(np.arange(1, n_ctx), size=n_cut, replace=False))
    starts = np.concatenate([[0], cuts]).astype(np.int32)
    lens = np.diff(np.concatenate([starts, [n_ctx]])).astype(np.int32)
    keep = rng.permutation(len(starts))[:int(rng.integers(1, len(starts) + 1))]
    with_self = bool(rng.integers(0, 2)) or len(keep) == 0
    ws = ("auto", None, "split")[int(rng.integers(0, 3))]
    return meta, hq, hkv, d, dtype, starts[keep], lens[keep], with_self, ws


@pytest.mark.parametrize("seed", range(64))
def test_random_case(seed):
    meta, hq, hkv, d, dtype, gs, gl, with_self, ws = draw_case(seed)
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, dtype, 1.0, gs, gl, self_block=with_self,
                            with_dout=True)
    scale = 1.0 / math.sqrt(d)
    dm = device_meta(meta, gs, gl)
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    ks, vs = dev(inp.k_self), dev(inp.v_self)
    ks64 = inp.k_self.f64 if with_self else None
    vs64 = inp.v_self.f64 if with_self else None
    f32 = dtype == "f32"
    case = (seed, meta.n_blk, meta.n_ctx, hq, hkv, d, dtype, len(gs), with_self, ws)

    # forward, one call over every listed chunk
    o, lse = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, out_dtype=torch.float32,
                                     workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, gs, gl, scale, ks64, vs64)
    if f32:
        assert rel_frob(host64(o), ro) <= 1e-5, case
        assert_lse_close(host64(lse), rl, 1e-5)
    else:
        assert np.abs(host64(o) - ro).max() <= 2e-2 and rel_frob(host64(o), ro) <= 1e-2, case
        assert_lse_close(host64(lse), rl, 1e-3)

    # one call per chunk (own-block term on the first), merged by the combine
    offs = np.concatenate([[0], np.cumsum(gl)]).astype(np.int64)
    parts_o, parts_l = [], []
    for c in range(len(gs)):
        mc = device_meta(meta, gs[c:c + 1], gl[c:c + 1])
        sl = slice(int(offs[c]), int(offs[c + 1]))
        po, pl = sxattn.sparse_xattn_fwd(q, k[sl].contiguous(), v[sl].contiguous(), mc, scale,
                                         ks if c == 0 else None, vs if c == 0 else None,
                                         out_dtype=torch.float32, workspace=ws)
        parts_o.append(po.reshape(-1, d))
        parts_l.append(pl.reshape(-1))
    co, cl = sxattn.lse_combine(torch.stack(parts_o), torch.stack(parts_l))
    torch.cuda.synchronize()
    tol_o = 1e-5 if f32 else 1e-2
    assert rel_frob(host64(co), ro.reshape(-1, d)) <= tol_o, case
    assert_lse_close(host64(cl), rl.reshape(-1), 1e-5 if f32 else 1e-3)

    # backward: GPU from the GPU forward, oracle from the oracle forward
    o_in, l_in = sxattn.sparse_xattn_fwd(q, k, v, dm, scale, ks, vs, workspace=ws)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk, dv, dks, dvs = sxattn.sparse_xattn_bwd(q, k, v, dm, scale, o_in, do, l_in, dq, ks, vs,
                                               workspace=ws)
    torch.cuda.synchronize()
    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale, ks64, vs64)
    tol = 1e-5 if f32 else 3e-2
    got = [(dq, r[0], "dq"), (dk, r[1], "dk"), (dv, r[2], "dv")]
    if with_self:
        got += [(dks, r[3], "dk_self"), (dvs, r[4], "dv_self")]
    for g, want, name in got:
        if not np.any(want):   # nothing reaches these entries: exact zeros
            assert not host64(g).any(), (name, case)
            continue
        err = rel_frob(host64(g), want)
        assert err <= tol, (name, err, case)
