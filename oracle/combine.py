"""Oracle: exact merge of attention partials from their log-sum-exp statistics.

Test infrastructure only; never used by the product path.

Split-KV combines the per-shard partial results using their normalisation
statistics so that the original attention is reconstructed exactly ("Split-KV
speeds diffusion drafter training...", section "Exchange the smaller side";
the abstract calls the method exact).  With lse_p the natural-log
log-sum-exp of partial p over its own keys and O_p its normalised output, the
full attention over the union of the keys is

    lse = log sum_p exp(lse_p)          O = sum_p exp(lse_p - lse) * O_p

computed here with the usual max shift m = max_p lse_p.  A partial with
lse_p = -inf has no allowed key: it carries no weight and its O_p is not read.
A row whose partials are all empty gets lse = -inf and O = 0.
"""

from __future__ import annotations

import numpy as np


def lse_combine(o_parts, lse_parts):
    """o_parts [P, R, d], lse_parts [P, R] -> (o [R, d], lse [R]) in float64."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    n_parts, rows, d = o_parts.shape
    out_o = np.zeros((rows, d))
    out_lse = np.full(rows, -np.inf)
    if n_parts == 0:
        return out_o, out_lse
    m = lse_parts.max(axis=0)
    live = np.isfinite(m)
    for r in np.flatnonzero(live):
        fin = np.isfinite(lse_parts[:, r])
        w = np.exp(lse_parts[fin, r] - m[r])
        tot = w.sum()
        out_lse[r] = m[r] + np.log(tot)
        out_o[r] = (w[:, None] * o_parts[fin, r, :]).sum(axis=0) / tot
    return out_o, out_lse
