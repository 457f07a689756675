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
