"""Shared test helpers: device upload of drawn inputs and error metrics."""

import numpy as np
import torch

from block_sparse_cross_anchor_amd import synth, sxattn


def dev(t, device="cuda"):
    """synth.Tensor (or None) -> device tensor with the exact same bits."""
    if t is None:
        return None
    if t.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(t.bits)).to(device)


def host64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def rel_frob(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))


def assert_lse_close(got, want, atol):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(want))
    fin = np.isfinite(want)
    assert np.all(np.isfinite(got[fin]))
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= atol, f"lse max abs error {err} > {atol}"


def device_meta(meta, chunk_gstart, chunk_len):
    return sxattn.Meta(meta.anchor, meta.sample_start, chunk_gstart, chunk_len)


def sub_blocks(meta, blocks):
    """Metadata restricted to a subset of blocks (blocks are independent)."""
    blocks = np.asarray(blocks)
    return synth.Meta(meta.lengths, meta.offsets, meta.anchor[blocks], meta.sample_start[blocks],
                      meta.n_ctx)


def token_rows(blocks, block=16):
    return np.concatenate([np.arange(b * block, (b + 1) * block) for b in blocks])


def readers(meta, g0, g1):
    """Blocks whose context interval [sample_start, anchor) meets the keys [g0, g1)."""
    return np.flatnonzero((meta.sample_start < g1) & (meta.anchor > g0))


def pick_windows(meta, chunk_gstart, chunk_len, rng, n, cap, width=64, tries=400):
    """Up to n key windows of `width` local rows inside single chunks, each read by 1 to
    `cap` blocks: (local row, global position, reader blocks)."""
    offs = np.concatenate([[0], np.cumsum(chunk_len)])
    out = []
    for _ in range(tries):
        c = int(rng.integers(0, len(chunk_gstart)))
        if chunk_len[c] < width:
            continue
        off = int(rng.integers(0, int(chunk_len[c]) - width + 1))
        g0 = int(chunk_gstart[c]) + off
        r = readers(meta, g0, g0 + width)
        if 1 <= r.size <= cap and all(g0 != w[1] for w in out):
            out.append((int(offs[c]) + off, g0, r))
            if len(out) == n:
                break
    return out


def head_rows(blocks, hq, block=16):
    """Rows of the flattened [n_q * hq] layout that belong to the given blocks."""
    t = token_rows(blocks, block)
    return (t[:, None] * hq + np.arange(hq)[None, :]).ravel()


def reader_pairs(meta, blocks):
    """Allowed context pairs per head of the given blocks (the oracle's work for them)."""
    blocks = np.asarray(blocks)
    return int(16 * (meta.anchor[blocks].astype(np.int64) - meta.sample_start[blocks]).sum())


def share_pairs(meta, blocks, chunk_gstart, chunk_len):
    """Allowed pairs per head of the given blocks over the listed chunks only."""
    b = np.asarray(blocks)
    lo = meta.sample_start[b].astype(np.int64)
    hi = meta.anchor[b].astype(np.int64)
    tot = 0
    for s, n in zip(np.asarray(chunk_gstart, np.int64), np.asarray(chunk_len, np.int64)):
        tot += int(16 * np.maximum(0, np.minimum(hi, s + n) - np.maximum(lo, s)).sum())
    return tot


def heavy_windows(meta, chunk_gstart, chunk_len, n, pair_budget, width=64, pairs_of=None):
    """Key windows with the most reading blocks: the n windows (aligned to `width`
    inside single chunks) read by the most blocks whose readers' oracle work
    (``pairs_of(blocks)``, default: their allowed pairs over the whole context) stays
    within pair_budget, and the window holding a sample start (read by every block of
    that sample) with the most readers within the budget.  Returns a list of
    (local row, global position, reader blocks), most readers first."""
    pairs_of = pairs_of or (lambda r: reader_pairs(meta, r))
    offs = np.concatenate([[0], np.cumsum(chunk_len)])
    cand = []
    for c in range(len(chunk_gstart)):
        for off in range(0, int(chunk_len[c]) - width + 1, width):
            g0 = int(chunk_gstart[c]) + off
            r = readers(meta, g0, g0 + width)
            if r.size and pairs_of(r) <= pair_budget:
                has_start = bool(np.any((meta.offsets >= g0) & (meta.offsets < g0 + width)))
                cand.append((r.size, has_start, int(offs[c]) + off, g0, r))
    cand.sort(key=lambda x: -x[0])
    out = [(l0, g0, r) for _, _, l0, g0, r in cand[:n]]
    starts = [x for x in cand if x[1]]
    if starts and all(starts[0][3] != w[1] for w in out):
        out.append((starts[0][2], starts[0][3], starts[0][4]))
    return out


def dkdv_split_tiles(meta, chunk_gstart, chunk_len, hq, hkv, n_shares, with_self,
                     setup_units=10, tile=256, step_rows=32):
    """A model of the load-balanced dK/dV schedule, used only to confirm what the tests
    cover: every kv head's list holds, per 256-key tile with hits, `setup_units` units
    plus one unit per hitting 32-row query step; n_shares workgroups take equal
    contiguous parts of the flattened list.  Returns, per tile (context tiles, then
    own-block tiles), the number of shares its steps span for kv head 0."""
    grp = hq // hkv
    ts = max(1, step_rows // grp)
    n_q = 16 * meta.n_blk
    gpos = np.concatenate([np.arange(s, s + n) for s, n in zip(chunk_gstart, chunk_len)]) \
        if len(chunk_gstart) else np.zeros(0, np.int64)
    lo = meta.sample_start.astype(np.int64)
    hi = meta.anchor.astype(np.int64)
    st_tok = np.arange(0, n_q, ts)
    b0, b1 = st_tok // 16, np.minimum(st_tok + ts, n_q) // 16
    b1 = np.minimum(b1, meta.n_blk - 1)
    hits = []
    for t0 in range(0, gpos.size, tile):
        kmin, kmax = int(gpos[t0:t0 + tile].min()), int(gpos[t0:t0 + tile].max())
        h = ((lo[b0] <= kmax) & (hi[b0] > kmin)) | ((lo[b1] <= kmax) & (hi[b1] > kmin))
        hits.append(int(h.sum()))
    if with_self:
        for t0 in range(0, n_q, tile):
            kmin, kmax = t0, min(t0 + tile, n_q) - 1
            h = ((16 * b0 <= kmax) & (16 * b0 + 16 > kmin)) | ((16 * b1 <= kmax) & (16 * b1 + 16 > kmin))
            hits.append(int(h.sum()))
    units = np.array([h + setup_units if h else 0 for h in hits], np.int64)
    prefix = np.concatenate([[0], np.cumsum(units)])
    tot = int(prefix[-1]) * hkv
    out = []
    for t, h in enumerate(hits):
        if h == 0:
            out.append(0)
            continue
        g0 = int(prefix[t]) + setup_units
        g1 = g0 + h
        j0 = ((g0 + 1) * n_shares - 1) // tot
        j1 = (g1 * n_shares - 1) // tot
        out.append(int(j1 - j0 + 1))
    return np.array(out)
