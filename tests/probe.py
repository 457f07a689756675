"""Mask-boundary probe with closed-form answers, for checks at full size.

With Q = 0 every allowed logit is 0, so attention is uniform over a block's allowed
keys: P = 1 / n_b with n_b = |allowed context keys| + 16 own-block keys.  The value
vectors are one-hot in a few probe columns, each column marking one class of
boundary position, so every output has a closed form that integer counting gives
(no oracle call, no floating-point attention on the host):

  forward   O[i, h, c] = hits_c(b) / n_b for the probe columns, 0 elsewhere;
            lse[i, h] = ln n_b.
  backward  dK = 0 (Q = 0);
            dV[j, g] = sum over blocks b that may read j of
                       (1 / n_b) sum_{i in b, h in g} dO[i, h];
            dQ[i, h] = (scale / n_b) sum_{j allowed} (dO[i, h] . V_j - D_ih) K_j,
                       D_ih = dO[i, h] . O[i, h].

Probe columns of the context values (global packed positions):
  0 sample starts (each block reads exactly one: its own sample's start),
  1 last token of every sample (no block may read its own sample's last token, and a
    block whose interval started one position early would read the previous one),
  2 anchor - 1 of every block (allowed for the block itself),
  3 anchors (never allowed for the block itself),
  4 chunk starts, 5 chunk ends - 1,
  6 about 1% random positions, 7 random positions at 64-key tile edges.
Own-block values: column 8 marks one random row of each block, column 9 every row.
An off-by-one at an interval end moves lse by about 1 / n_b and the hit count of some
column by one.
"""

from __future__ import annotations

import numpy as np

from block_sparse_cross_anchor_amd import synth

N_COLS = 10
ONE_BF16 = int(synth.f32_to_bf16_bits(np.ones(1, np.float32))[0])


def positions(meta, chunk_size, seed):
    """Probe positions of columns 0..7 (sorted unique int64 arrays)."""
    rng = np.random.default_rng(seed)
    n = meta.n_ctx
    ends = meta.offsets + meta.lengths
    cs = np.arange(0, n, chunk_size, dtype=np.int64)
    ce = np.minimum(cs + chunk_size, n) - 1
    rand = rng.choice(n, size=max(1, n // 100), replace=False)
    tiles = np.arange(0, n, 64, dtype=np.int64)
    edge = np.concatenate([tiles, tiles + 63])
    edge = rng.choice(edge[edge < n], size=max(1, n // 256), replace=False)
    cols = [meta.offsets, ends - 1, meta.anchor.astype(np.int64) - 1, meta.anchor.astype(np.int64),
            cs, ce, rand, edge]
    return [np.unique(np.asarray(c, np.int64)) for c in cols]


def self_rows(n_blk, seed):
    """Row (0..15) of each block marked in own-block column 8."""
    return np.random.default_rng(seed + 1).integers(0, 16, size=n_blk)


def inputs(seed, meta, hq, hkv, d, chunk_gstart, chunk_len, chunk_size):
    """synth.Inputs for the probe on the given local chunks: Q = 0, K random, V
    one-hot at the probe positions, k_self random, v_self one-hot, dO ~ N(0, 1)."""
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "bf16", 1.0 / np.sqrt(d), chunk_gstart,
                            chunk_len, with_dout=True)
    inp.q = synth.Tensor(np.zeros_like(inp.q.bits), "bf16")
    gpos = synth.chunk_rows(chunk_gstart, chunk_len)
    vb = np.zeros(inp.v.bits.shape, np.uint16)
    for c, pos in enumerate(positions(meta, chunk_size, seed)):
        vb[np.isin(gpos, pos), :, c] = ONE_BF16
    inp.v = synth.Tensor(vb, "bf16")
    vs = np.zeros(inp.v_self.bits.shape, np.uint16)
    r = self_rows(meta.n_blk, seed)
    vs[16 * np.arange(meta.n_blk) + r, :, 8] = ONE_BF16
    vs[:, :, 9] = ONE_BF16
    inp.v_self = synth.Tensor(vs, "bf16")
    return inp


def _in_share(pos, gs, gl):
    ok = np.zeros(pos.shape, bool)
    for s, n in zip(gs, gl):
        ok |= (pos >= s) & (pos < s + n)
    return ok


def counts(meta, gs, gl):
    """n_b over the listed chunks (own block included) as int64 [n_blk]."""
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    n = np.full(meta.n_blk, 16, np.int64)
    for s, ln in zip(np.asarray(gs, np.int64), np.asarray(gl, np.int64)):
        n += np.maximum(0, np.minimum(hi, s + ln) - np.maximum(lo, s))
    return n


def forward(meta, gs, gl, chunk_size, seed):
    """Expected (n_b, hits [n_blk, N_COLS]) of the probe over the listed chunks."""
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    hits = np.zeros((meta.n_blk, N_COLS), np.int64)
    for c, pos in enumerate(positions(meta, chunk_size, seed)):
        pos = pos[_in_share(pos, gs, gl)]
        hits[:, c] = np.searchsorted(pos, hi, "left") - np.searchsorted(pos, lo, "left")
    hits[:, 8] = 1
    hits[:, 9] = 16
    return counts(meta, gs, gl), hits


def dv_context(meta, inp, gs, gl, hq, hkv):
    """Expected float64 dV [n_loc, hkv, d] of the local rows (chunks back to back)."""
    n_b = counts(meta, gs, gl)
    grp = hq // hkv
    do = inp.dout.f64.reshape(meta.n_blk, 16, hkv, grp, -1)
    cb = do.sum(axis=(1, 3)) / n_b[:, None, None]            # [n_blk, hkv, d]
    out = []
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    for s, ln in zip(np.asarray(gs, np.int64), np.asarray(gl, np.int64)):
        diff = np.zeros((ln + 1,) + cb.shape[1:])
        nread = np.zeros(ln + 1, np.int64)
        a = np.clip(lo - s, 0, ln)
        e = np.clip(hi - s, 0, ln)
        live = a < e
        np.add.at(diff, a[live], cb[live])
        np.add.at(diff, e[live], -cb[live])
        np.add.at(nread, a[live], 1)
        np.add.at(nread, e[live], -1)
        dv = np.cumsum(diff, axis=0)[:ln]
        dv[np.cumsum(nread)[:ln] == 0] = 0.0   # keys no block reads: exactly zero
        out.append(dv)
    return np.concatenate(out) if out else np.zeros((0,) + cb.shape[1:])


def dv_self(meta, inp, gs, gl, hq, hkv):
    """Expected float64 own-block dV [n_q, hkv, d]: every row of block b gets c_b."""
    n_b = counts(meta, gs, gl)
    grp = hq // hkv
    do = inp.dout.f64.reshape(meta.n_blk, 16, hkv, grp, -1)
    cb = do.sum(axis=(1, 3)) / n_b[:, None, None]
    return np.repeat(cb, 16, axis=0)


def dq(meta, inp, gs, gl, hq, hkv, scale, chunk_size, seed):
    """Expected float64 dQ [n_q, hq, d] of the probe over the listed chunks (own block
    included), from the exact probe output."""
    n_blk = meta.n_blk
    grp = hq // hkv
    n_b, hits = forward(meta, gs, gl, chunk_size, seed)
    d = inp.k.shape[-1]
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    k = inp.k.f64                                            # local rows
    ks = inp.k_self.f64.reshape(n_blk, 16, hkv, d)
    # sum of K over each block's allowed keys, and over its probe keys of each column
    sk_all = np.zeros((n_blk, hkv, d))
    off = 0
    for s, ln in zip(np.asarray(gs, np.int64), np.asarray(gl, np.int64)):
        pre = np.concatenate([np.zeros((1, hkv, d)), np.cumsum(k[off:off + ln], axis=0)])
        a = np.clip(lo - s, 0, ln)
        e = np.clip(hi - s, 0, ln)
        sk_all += pre[np.maximum(a, e)] - pre[a]
        off += ln
    gpos = synth.chunk_rows(gs, gl)
    sk_c = np.zeros((N_COLS, n_blk, hkv, d))
    for c, pos in enumerate(positions(meta, chunk_size, seed)):
        rows = np.flatnonzero(np.isin(gpos, pos))
        if rows.size:
            p = gpos[rows]
            m = (lo[:, None] <= p[None, :]) & (p[None, :] < hi[:, None])
            sk_c[c] = np.einsum("bp,pgd->bgd", m.astype(np.float64), k[rows])
    r = self_rows(n_blk, seed)
    sk_c[8] = ks[np.arange(n_blk), r]
    sk_c[9] = ks.sum(axis=1)
    sk_all += ks.sum(axis=1)
    do = inp.dout.f64.reshape(n_blk, 16, hkv, grp, d)
    o_exact = hits / n_b[:, None]                            # [n_blk, N_COLS]
    dlt = np.einsum("btgjc,bc->btgj", do[..., :N_COLS], o_exact)
    acc = np.einsum("btgjc,cbgd->btgjd", do[..., :N_COLS], sk_c)
    acc -= dlt[..., None] * sk_all[:, None, :, None, :]
    acc *= (scale / n_b)[:, None, None, None, None]
    return acc.reshape(n_blk * 16, hq, d)
