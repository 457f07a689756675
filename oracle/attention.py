"""Oracle: anchor-masked block-sparse cross-attention, forward and backward (float64).

Test infrastructure only (see the package docstring); never used by the product path.

The mask is the one stated on the Split-KV page "Split-KV speeds diffusion
drafter training by keeping long-context data local", section "Why short
queries change the problem": each draft block opened by an anchor attends to
the preceding context of its own sample and to every token of its own block.
Readings taken where the page is silent (all listed in the design notes):

* the context a block reads = global packed positions j with
  sample_start[b] <= j < anchor[b] (same sample, strictly before the anchor;
  the anchor position itself is excluded);
* the block's own tokens = its draft tokens, whose keys and values are supplied
  separately (``k_self``/``v_self``, rows b*B..b*B+B-1), attended
  bidirectionally (all of them, no causal order);
* grouped-query heads: query head h reads kv head h // (hq // hkv);
* logits are ``scale * <q, k>`` with ``scale`` taken as a float32 value; the
  log-sum-exp is natural-log and includes the scale; a row with no allowed key
  has lse = -inf and output 0.

The local key/value buffer holds the listed context chunks back to back; chunk
i covers global positions [chunk_gstart[i], chunk_gstart[i] + chunk_len[i]).
Each call yields the partial result over its own chunks (section "Exchange the
smaller side": keys and values stay local and every device evaluates all
queries against its shard); partials are merged by ``oracle.combine``.

The backward follows from differentiating that definition; given the merged
output O and merged lse of the full attention it needs no forward state:
P = exp(s - lse), D = rowsum(dO * O), dS = P * (dO V^T - D),
dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, each summed over the query
heads that share a kv head.
"""

from __future__ import annotations

import numpy as np


def f32_scale(scale: float) -> float:
    """The softmax scale as the float32 value the device receives."""
    return float(np.float32(scale))


def allowed_local_ranges(lo: int, hi: int, chunk_gstart, chunk_len):
    """Local row ranges [a, b) of the chunks' keys at global positions in [lo, hi)."""
    out, off = [], 0
    for gs, n in zip(chunk_gstart, chunk_len):
        gs, n = int(gs), int(n)
        a, b = max(lo, gs), min(hi, gs + n)
        if a < b:
            out.append((off + a - gs, off + b - gs))
        off += n
    return out


def allowed_local_rows(lo: int, hi: int, chunk_gstart, chunk_len) -> np.ndarray:
    r = allowed_local_ranges(lo, hi, chunk_gstart, chunk_len)
    if not r:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(a, b) for a, b in r])


def _block_keys(b, g, block, k, v, idx, k_self, v_self):
    kk, vv = k[idx, g, :], v[idx, g, :]
    if k_self is not None:
        rows = slice(b * block, (b + 1) * block)
        kk = np.concatenate([kk, k_self[rows, g, :]], axis=0)
        vv = np.concatenate([vv, v_self[rows, g, :]], axis=0)
    return kk, vv


def sparse_xattn_fwd(q, k, v, anchor, sample_start, chunk_gstart, chunk_len, scale,
                     k_self=None, v_self=None, block: int = 16):
    """Partial forward over one call's chunks (plus the own-block term if given).

    q [n_q, hq, d]; k, v [n_loc, hkv, d] (the chunks back to back); k_self, v_self
    [n_q, hkv, d] or None.  Returns (o [n_q, hq, d], lse [n_q, hq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k_self is not None:
        k_self = np.asarray(k_self, dtype=np.float64)
        v_self = np.asarray(v_self, dtype=np.float64)
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    sc = f32_scale(scale)
    n_blk = len(anchor)
    assert n_q == n_blk * block
    o = np.zeros((n_q, hq, d))
    lse = np.full((n_q, hq), -np.inf)
    for b in range(n_blk):
        idx = allowed_local_rows(int(sample_start[b]), int(anchor[b]), chunk_gstart, chunk_len)
        rows = slice(b * block, (b + 1) * block)
        for g in range(hkv):
            kk, vv = _block_keys(b, g, block, k, v, idx, k_self, v_self)
            if kk.shape[0] == 0:
                continue
            heads = slice(g * grp, (g + 1) * grp)
            qq = q[rows, heads, :].reshape(block * grp, d)
            s = sc * (qq @ kk.T)
            m = s.max(axis=1)
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            o[rows, heads, :] = ((e @ vv) / l[:, None]).reshape(block, grp, d)
            lse[rows, heads] = (m + np.log(l)).reshape(block, grp)
    return o, lse


def sparse_xattn_bwd(q, k, v, o, dout, lse, anchor, sample_start, chunk_gstart, chunk_len,
                     scale, k_self=None, v_self=None, block: int = 16):
    """Backward contribution of one call's chunks (plus the own-block term if given).

    ``o`` and ``lse`` are the merged (full-attention) output and log-sum-exp.
    Returns (dq, dk, dv, dk_self, dv_self): dq is this call's contribution to the
    query gradient (callers sum it over calls); dk, dv cover the local rows;
    dk_self, dv_self are None when no own-block term is given.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    if k_self is not None:
        k_self = np.asarray(k_self, dtype=np.float64)
        v_self = np.asarray(v_self, dtype=np.float64)
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    sc = f32_scale(scale)
    n_blk = len(anchor)
    delta = (dout * o).sum(axis=-1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dks = np.zeros_like(k_self) if k_self is not None else None
    dvs = np.zeros_like(v_self) if k_self is not None else None
    for b in range(n_blk):
        idx = allowed_local_rows(int(sample_start[b]), int(anchor[b]), chunk_gstart, chunk_len)
        n_ctx_keys = idx.shape[0]
        rows = slice(b * block, (b + 1) * block)
        for g in range(hkv):
            kk, vv = _block_keys(b, g, block, k, v, idx, k_self, v_self)
            if kk.shape[0] == 0:
                continue
            heads = slice(g * grp, (g + 1) * grp)
            qq = q[rows, heads, :].reshape(block * grp, d)
            dd = dout[rows, heads, :].reshape(block * grp, d)
            L = lse[rows, heads].reshape(-1)
            Dr = delta[rows, heads].reshape(-1)
            s = sc * (qq @ kk.T)
            fin = np.isfinite(L)
            p = np.zeros_like(s)
            p[fin] = np.exp(s[fin] - L[fin, None])
            dv_b = p.T @ dd
            dp = dd @ vv.T
            ds = p * (dp - Dr[:, None])
            dq[rows, heads, :] += (sc * (ds @ kk)).reshape(block, grp, d)
            dk_b = sc * (ds.T @ qq)
            dk[idx, g, :] += dk_b[:n_ctx_keys]
            dv[idx, g, :] += dv_b[:n_ctx_keys]
            if k_self is not None:
                dks[rows, g, :] += dk_b[n_ctx_keys:]
                dvs[rows, g, :] += dv_b[n_ctx_keys:]
    return dq, dk, dv, dks, dvs
