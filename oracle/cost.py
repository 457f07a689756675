"""Oracle: per-chunk realised attention cost, by brute force.

Test infrastructure only; never used by the product path.

The planner prices each context chunk by the attention work that lands on it;
since every device holds the metadata of all query blocks, each device can count
that work for every chunk ("Split-KV speeds diffusion drafter training...",
section "Balance actual attention work").  Reading taken here: the cost of a chunk is the number of (query token, context
key) pairs inside the chunk that the anchor mask allows, for one head (all
heads cost the same); own-block pairs are not context work and are not
counted.  Chunks are the contiguous fixed-size spans
[c*chunk_size, min((c+1)*chunk_size, n_ctx)) of the packed context.

The count is taken literally: the mask predicate
sample_start[b(i)] <= j < anchor[b(i)] is evaluated for every query token i
and every key position j of the chunk and the true entries are counted.
"""

from __future__ import annotations

import numpy as np


def _token_bounds(anchor, sample_start, block):
    lo = np.repeat(np.asarray(sample_start, dtype=np.int64), block)
    hi = np.repeat(np.asarray(anchor, dtype=np.int64), block)
    return lo, hi


def chunk_cost_one(anchor, sample_start, c: int, chunk_size: int, n_ctx: int,
                   block: int = 16) -> int:
    """Allowed (query token, key) pairs with the key in chunk c."""
    lo, hi = _token_bounds(anchor, sample_start, block)
    j = np.arange(c * chunk_size, min((c + 1) * chunk_size, n_ctx), dtype=np.int64)
    allowed = (lo[:, None] <= j[None, :]) & (j[None, :] < hi[:, None])
    return int(np.count_nonzero(allowed))


def chunk_cost(anchor, sample_start, n_ctx: int, chunk_size: int, block: int = 16,
               chunks=None) -> np.ndarray:
    """int64 cost of every chunk (or of the listed chunk indices)."""
    n_chunk = -(-n_ctx // chunk_size)
    which = range(n_chunk) if chunks is None else chunks
    return np.asarray([chunk_cost_one(anchor, sample_start, int(c), chunk_size, n_ctx, block)
                       for c in which], dtype=np.int64)


def total_pairs(anchor, sample_start, n_ctx: int, block: int = 16) -> int:
    """Allowed (query token, key) pairs over the whole context, by brute force."""
    lo, hi = _token_bounds(anchor, sample_start, block)
    j = np.arange(n_ctx, dtype=np.int64)
    return int(sum(np.count_nonzero((lo[i] <= j) & (j < hi[i])) for i in range(lo.shape[0])))
