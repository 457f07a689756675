"""Textbook dense masked softmax attention, used only to pin the oracle.

Test infrastructure only; never used by the product path.

It materialises the full boolean mask over every (query, key) pair from the
predicate of "Split-KV speeds diffusion drafter training...", section "Why
short queries change the problem" (own-sample context before the anchor, plus
the block's own tokens), sets masked logits to -inf and calls scipy's
``logsumexp``/``softmax``.  It shares no code with ``oracle.attention``.
"""

from __future__ import annotations

import numpy as np
from scipy.special import logsumexp, softmax


def dense_mask(anchor, sample_start, chunk_gstart, chunk_len, with_self: bool,
               block: int = 16) -> np.ndarray:
    """[n_q, n_loc (+ n_q)] mask; columns are the local context rows, then the
    n_q own-block key rows when ``with_self``."""
    gpos = [np.arange(int(s), int(s) + int(n)) for s, n in zip(chunk_gstart, chunk_len)]
    gpos = np.concatenate(gpos) if gpos else np.zeros(0, dtype=np.int64)
    n_q = len(anchor) * block
    tok_lo = np.repeat(np.asarray(sample_start, np.int64), block)
    tok_hi = np.repeat(np.asarray(anchor, np.int64), block)
    ctx = (tok_lo[:, None] <= gpos[None, :]) & (gpos[None, :] < tok_hi[:, None])
    if not with_self:
        return ctx
    blk = np.arange(n_q) // block
    own = blk[:, None] == blk[None, :]
    return np.concatenate([ctx, own], axis=1)


def dense_fwd(q, kcat, vcat, mask, scale):
    """q [n_q, hq, d]; kcat, vcat [n_keys, hkv, d]; mask [n_q, n_keys]."""
    q = np.asarray(q, np.float64)
    kcat = np.asarray(kcat, np.float64)
    vcat = np.asarray(vcat, np.float64)
    n_q, hq, d = q.shape
    hkv = kcat.shape[1]
    sc = float(np.float32(scale))
    o = np.zeros((n_q, hq, d))
    lse = np.full((n_q, hq), -np.inf)
    for h in range(hq):
        g = h * hkv // hq
        s = sc * (q[:, h, :] @ kcat[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        live = mask.any(axis=1)
        lse[live, h] = logsumexp(s[live], axis=1)
        p = softmax(s[live], axis=1)
        o[live, h, :] = p @ vcat[:, g, :]
    return o, lse
