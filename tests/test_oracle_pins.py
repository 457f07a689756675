"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* forward: a textbook dense masked softmax (scipy logsumexp/softmax over a full
  boolean mask built from the predicate), special cases with closed forms
  (Q = 0 gives uniform attention; a single allowed key returns its value), a
  mask-boundary probe, and row sums of the attention probabilities;
* combine: split-then-combine equals unsplit for arbitrary partitions and
  orders, P = 1 is the identity, combining a partial with itself adds ln 2;
* backward: torch autograd in float64 on the dense formulation, central finite
  differences, and the sum of per-chunk calls equals the unsplit call;
* cost / LPT: hand-worked golden fixtures, closed-form totals, properties.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_case(seed, n_ctx=260, len_lo=40, len_hi=120, n_anchor=5, hq=4, hkv=2, d=8,
              chunk_size=64, perm=False, self_block=True, std=1.0):
    meta = synth.draw_meta(seed, n_ctx, len_lo, len_hi, n_anchor)
    gs, gl = synth.contiguous_chunks(n_ctx, chunk_size)
    if perm:
        p = np.random.default_rng(seed + 7).permutation(len(gs))
        gs, gl = gs[p], gl[p]
    inp = synth.draw_inputs(seed, meta, hq, hkv, d, "f32", std, gs, gl, self_block=self_block,
                            with_dout=True)
    return meta, inp


def kcat_vcat(inp):
    k, v = inp.k.f64, inp.v.f64
    if inp.k_self is not None:
        k = np.concatenate([k, inp.k_self.f64], axis=0)
        v = np.concatenate([v, inp.v_self.f64], axis=0)
    return k, v


# ----------------------------------------------------------------------------- forward

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("self_block", [True, False])
def test_fwd_equals_dense_softmax(seed, self_block):
    meta, inp = tiny_case(seed, perm=(seed % 2 == 1), self_block=self_block,
                          chunk_size=[64, 50, 97][seed % 3])
    scale = 1.0 / math.sqrt(8)
    o, lse = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, inp.chunk_gstart, inp.chunk_len, scale,
                                     None if inp.k_self is None else inp.k_self.f64,
                                     None if inp.v_self is None else inp.v_self.f64)
    mask = oracle.dense_mask(meta.anchor, meta.sample_start, inp.chunk_gstart, inp.chunk_len,
                             self_block)
    k, v = kcat_vcat(inp)
    o2, lse2 = oracle.dense_fwd(inp.q.f64, k, v, mask, scale)
    np.testing.assert_allclose(o, o2, atol=1e-12, rtol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lse2))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lse2[fin], atol=1e-12, rtol=1e-12)


def test_fwd_on_a_subset_of_chunks_has_empty_rows():
    """A call holding only late chunks leaves early blocks with no allowed key."""
    meta, inp = tiny_case(3, chunk_size=32, self_block=False)
    keep = [len(inp.chunk_gstart) - 1]
    gs, gl = inp.chunk_gstart[keep], inp.chunk_len[keep]
    rows = synth.chunk_rows(gs, gl)
    k = synth.draw_context(3, 2, rows, 2, 8, 1.0, "f32").f64
    v = synth.draw_context(3, 3, rows, 2, 8, 1.0, "f32").f64
    o, lse = oracle.sparse_xattn_fwd(inp.q.f64, k, v, meta.anchor, meta.sample_start, gs, gl, 0.3)
    mask = oracle.dense_mask(meta.anchor, meta.sample_start, gs, gl, False)
    empty = ~mask.any(axis=1)
    assert empty.any()
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0)
    o2, lse2 = oracle.dense_fwd(inp.q.f64, k, v, mask, 0.3)
    np.testing.assert_allclose(o, o2, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_probability_rows_sum_to_one(seed):
    meta, inp = tiny_case(seed)
    scale = 0.7
    o, lse = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, inp.chunk_gstart, inp.chunk_len, scale,
                                     inp.k_self.f64, inp.v_self.f64)
    mask = oracle.dense_mask(meta.anchor, meta.sample_start, inp.chunk_gstart, inp.chunk_len, True)
    k, _ = kcat_vcat(inp)
    sc = float(np.float32(scale))
    for h in range(4):
        s = sc * inp.q.f64[:, h, :] @ k[:, h // 2, :].T
        p = np.where(mask, np.exp(s - lse[:, h:h + 1]), 0.0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


def _allowed_count(meta, gs, gl, i, block=16, self_block=True):
    """Count allowed keys of query token i by walking every local position."""
    b = i // block
    n = 0
    for s, ln in zip(gs, gl):
        for j in range(int(s), int(s) + int(ln)):
            if meta.sample_start[b] <= j < meta.anchor[b]:
                n += 1
    return n + (block if self_block else 0)


@pytest.mark.parametrize("seed", range(3))
def test_zero_queries_give_uniform_attention(seed):
    """Q = 0: every allowed logit is 0, so lse = ln(#allowed) and O = mean of allowed V."""
    meta, inp = tiny_case(seed, perm=True, chunk_size=45)
    q0 = np.zeros_like(inp.q.f64)
    o, lse = oracle.sparse_xattn_fwd(q0, inp.k.f64, inp.v.f64, meta.anchor, meta.sample_start,
                                     inp.chunk_gstart, inp.chunk_len, 1.0, inp.k_self.f64,
                                     inp.v_self.f64)
    gpos = synth.chunk_rows(inp.chunk_gstart, inp.chunk_len)
    for i in range(q0.shape[0]):
        n = _allowed_count(meta, inp.chunk_gstart, inp.chunk_len, i)
        np.testing.assert_allclose(lse[i], math.log(n), atol=1e-13)
        b = i // 16
        sel = (meta.sample_start[b] <= gpos) & (gpos < meta.anchor[b])
        for h in range(4):
            g = h // 2
            tot = inp.v.f64[sel, g, :].sum(axis=0) + inp.v_self.f64[16 * b:16 * b + 16, g, :].sum(axis=0)
            np.testing.assert_allclose(o[i, h], tot / n, atol=1e-12)


def test_single_allowed_key_returns_its_value():
    """anchor = sample_start + 1 and no own-block term: the only key is the sample start."""
    anchor = np.array([1, 41], np.int32)
    start = np.array([0, 40], np.int32)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((32, 2, 4))
    k = rng.standard_normal((64, 1, 4))
    v = rng.standard_normal((64, 1, 4))
    o, lse = oracle.sparse_xattn_fwd(q, k, v, anchor, start, [0], [64], 0.5)
    for i in range(32):
        j = 0 if i < 16 else 40
        for h in range(2):
            np.testing.assert_allclose(o[i, h], v[j, 0], atol=1e-15)
            np.testing.assert_allclose(lse[i, h], float(np.float32(0.5)) * q[i, h] @ k[j, 0],
                                       atol=1e-13)


def test_mask_boundary_probe():
    """Q = 0, V channel 0 = 1 only at probe positions (sample start, anchor - 1, anchor,
    chunk edges): O[i, h, 0] = (#probes strictly inside the allowed set) / #allowed."""
    meta, inp = tiny_case(11, chunk_size=40, self_block=False, perm=True)
    gpos = synth.chunk_rows(inp.chunk_gstart, inp.chunk_len)
    probes = set()
    for b in range(meta.n_blk):
        probes |= {int(meta.sample_start[b]), int(meta.anchor[b]) - 1, int(meta.anchor[b])}
    for s, n in zip(inp.chunk_gstart, inp.chunk_len):
        probes |= {int(s), int(s) + int(n) - 1}
    v = np.zeros_like(inp.v.f64)
    for r, j in enumerate(gpos):
        if int(j) in probes:
            v[r, :, 0] = 1.0
    o, lse = oracle.sparse_xattn_fwd(np.zeros_like(inp.q.f64), inp.k.f64, v, meta.anchor,
                                     meta.sample_start, inp.chunk_gstart, inp.chunk_len, 1.0)
    for i in range(inp.q.shape[0]):
        b = i // 16
        allowed = [j for j in range(meta.n_ctx) if meta.sample_start[b] <= j < meta.anchor[b]]
        hit = sum(1 for j in allowed if j in probes)
        np.testing.assert_allclose(o[i, :, 0], hit / len(allowed), atol=1e-14)
        np.testing.assert_allclose(lse[i], math.log(len(allowed)), atol=1e-13)


# ----------------------------------------------------------------------------- combine

def _chunked_partials(meta, inp, groups, scale, self_group=0):
    """Run the oracle per group of chunk indices (own-block term on one group)."""
    outs = []
    for gi, grp in enumerate(groups):
        gs, gl = inp.chunk_gstart[grp], inp.chunk_len[grp]
        all_rows = synth.chunk_rows(inp.chunk_gstart, inp.chunk_len)
        offs = np.concatenate([[0], np.cumsum(inp.chunk_len)])
        rows = np.concatenate([np.arange(offs[c], offs[c + 1]) for c in grp]) if len(grp) else \
            np.zeros(0, np.int64)
        assert np.array_equal(all_rows[rows], synth.chunk_rows(gs, gl))
        ks = inp.k_self.f64 if gi == self_group else None
        vs = inp.v_self.f64 if gi == self_group else None
        outs.append(oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64[rows], inp.v.f64[rows],
                                            meta.anchor, meta.sample_start, gs, gl, scale, ks, vs))
    return outs


@pytest.mark.parametrize("seed", range(5))
def test_split_then_combine_equals_unsplit(seed):
    meta, inp = tiny_case(seed, chunk_size=23)
    n = len(inp.chunk_gstart)
    rng = np.random.default_rng(100 + seed)
    n_parts = int(rng.integers(2, 6))
    lab = rng.integers(0, n_parts, size=n)
    groups = [np.flatnonzero(lab == p) for p in range(n_parts)]
    parts = _chunked_partials(meta, inp, groups, 0.4, self_group=int(rng.integers(0, n_parts)))
    order = rng.permutation(n_parts)
    o_parts = np.stack([parts[p][0] for p in order]).reshape(n_parts, -1, 8)
    l_parts = np.stack([parts[p][1] for p in order]).reshape(n_parts, -1)
    o, lse = oracle.lse_combine(o_parts, l_parts)
    o_ref, lse_ref = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                             meta.sample_start, inp.chunk_gstart, inp.chunk_len,
                                             0.4, inp.k_self.f64, inp.v_self.f64)
    np.testing.assert_allclose(o, o_ref.reshape(-1, 8), atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.reshape(-1), atol=1e-12)


def test_combine_identity_self_and_empty():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((1, 7, 3))
    lse = rng.uniform(-3, 3, (1, 7))
    lse[0, 2] = -np.inf
    o[0, 2] = 0.0
    co, cl = oracle.lse_combine(o, lse)
    np.testing.assert_array_equal(cl, lse[0])
    np.testing.assert_allclose(co, o[0], atol=1e-15)
    co2, cl2 = oracle.lse_combine(np.concatenate([o, o]), np.concatenate([lse, lse]))
    fin = np.isfinite(lse[0])
    np.testing.assert_allclose(cl2[fin], lse[0, fin] + math.log(2), atol=1e-14)
    np.testing.assert_allclose(co2, o[0], atol=1e-15)
    assert np.isneginf(cl2[2]) and np.all(co2[2] == 0)
    # an empty partial's O is never read, even if it holds garbage
    o3 = np.concatenate([o, np.full_like(o, np.nan)])
    l3 = np.concatenate([lse, np.full_like(lse, -np.inf)])
    co3, cl3 = oracle.lse_combine(o3, l3)
    np.testing.assert_allclose(co3, o[0], atol=1e-15)


def test_combine_is_associative():
    rng = np.random.default_rng(9)
    o = rng.standard_normal((5, 11, 4))
    lse = rng.uniform(-5, 5, (5, 11))
    lse[1, 3] = lse[4, 3] = -np.inf
    full_o, full_l = oracle.lse_combine(o, lse)
    a_o, a_l = oracle.lse_combine(o[:2], lse[:2])
    b_o, b_l = oracle.lse_combine(o[2:], lse[2:])
    c_o, c_l = oracle.lse_combine(np.stack([a_o, b_o]), np.stack([a_l, b_l]))
    np.testing.assert_allclose(c_o, full_o, atol=1e-13)
    np.testing.assert_allclose(c_l, full_l, atol=1e-13)


def test_combine_closed_form_two_partials():
    """Two partials with lse a, b and outputs x, y: weights are logistic functions of a - b."""
    a, b = 1.25, -0.5
    x, y = np.array([[2.0, -1.0]]), np.array([[0.5, 4.0]])
    co, cl = oracle.lse_combine(np.stack([x, y]), np.array([[a], [b]]))
    wa = 1.0 / (1.0 + math.exp(b - a))
    np.testing.assert_allclose(co[0], wa * x[0] + (1 - wa) * y[0], atol=1e-15)
    np.testing.assert_allclose(cl[0], math.log(math.exp(a) + math.exp(b)), atol=1e-15)


# ----------------------------------------------------------------------------- backward

def _dense_torch_grads(meta, inp, scale, self_block=True):
    q = torch.tensor(inp.q.f64, requires_grad=True)
    kc, vc = kcat_vcat(inp) if self_block else (inp.k.f64, inp.v.f64)
    k = torch.tensor(kc, requires_grad=True)
    v = torch.tensor(vc, requires_grad=True)
    mask = torch.tensor(oracle.dense_mask(meta.anchor, meta.sample_start, inp.chunk_gstart,
                                          inp.chunk_len, self_block))
    hq, hkv = q.shape[1], k.shape[1]
    sc = float(np.float32(scale))
    outs = []
    for h in range(hq):
        g = h * hkv // hq
        s = sc * q[:, h, :] @ k[:, g, :].T
        s = s.masked_fill(~mask, float("-inf"))
        p = torch.softmax(s, dim=1)
        outs.append(p @ v[:, g, :])
    o = torch.stack(outs, dim=1)
    do = torch.tensor(inp.dout.f64)
    (o * do).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed", range(4))
def test_bwd_equals_torch_autograd_and_sums_over_chunks(seed):
    meta, inp = tiny_case(seed, chunk_size=37, perm=(seed % 2 == 0))
    scale = 0.45
    o, lse = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, inp.chunk_gstart, inp.chunk_len, scale,
                                     inp.k_self.f64, inp.v_self.f64)
    o_t, dq_t, dk_t, dv_t = _dense_torch_grads(meta, inp, scale)
    np.testing.assert_allclose(o, o_t, atol=1e-12)
    n_loc = inp.k.shape[0]
    # unsplit call
    dq, dk, dv, dks, dvs = oracle.sparse_xattn_bwd(
        inp.q.f64, inp.k.f64, inp.v.f64, o, inp.dout.f64, lse, meta.anchor, meta.sample_start,
        inp.chunk_gstart, inp.chunk_len, scale, inp.k_self.f64, inp.v_self.f64)
    np.testing.assert_allclose(dq, dq_t, atol=1e-11)
    np.testing.assert_allclose(dk, dk_t[:n_loc], atol=1e-11)
    np.testing.assert_allclose(dv, dv_t[:n_loc], atol=1e-11)
    np.testing.assert_allclose(dks, dk_t[n_loc:], atol=1e-11)
    np.testing.assert_allclose(dvs, dv_t[n_loc:], atol=1e-11)
    # one call per chunk, own-block term on the first call, dq summed
    offs = np.concatenate([[0], np.cumsum(inp.chunk_len)])
    dq_sum = np.zeros_like(dq)
    for c in range(len(inp.chunk_gstart)):
        rows = np.arange(offs[c], offs[c + 1])
        r = oracle.sparse_xattn_bwd(
            inp.q.f64, inp.k.f64[rows], inp.v.f64[rows], o, inp.dout.f64, lse, meta.anchor,
            meta.sample_start, inp.chunk_gstart[c:c + 1], inp.chunk_len[c:c + 1], scale,
            inp.k_self.f64 if c == 0 else None, inp.v_self.f64 if c == 0 else None)
        dq_sum += r[0]
        np.testing.assert_allclose(r[1], dk_t[rows], atol=1e-11)
        np.testing.assert_allclose(r[2], dv_t[rows], atol=1e-11)
    np.testing.assert_allclose(dq_sum, dq_t, atol=1e-11)


def test_bwd_central_finite_differences():
    meta, inp = tiny_case(21, n_ctx=150, len_lo=40, len_hi=80, n_anchor=3, hq=2, hkv=1, d=4,
                          chunk_size=50)
    scale = 0.6
    args = dict(anchor=meta.anchor, sample_start=meta.sample_start,
                chunk_gstart=inp.chunk_gstart, chunk_len=inp.chunk_len, scale=scale)
    tensors = {"q": inp.q.f64.copy(), "k": inp.k.f64.copy(), "v": inp.v.f64.copy(),
               "k_self": inp.k_self.f64.copy(), "v_self": inp.v_self.f64.copy()}
    do = inp.dout.f64

    def loss(t):
        o, _ = oracle.sparse_xattn_fwd(t["q"], t["k"], t["v"], k_self=t["k_self"],
                                       v_self=t["v_self"], **args)
        return float((o * do).sum())

    o, lse = oracle.sparse_xattn_fwd(tensors["q"], tensors["k"], tensors["v"],
                                     k_self=tensors["k_self"], v_self=tensors["v_self"], **args)
    grads = dict(zip(["q", "k", "v", "k_self", "v_self"], oracle.sparse_xattn_bwd(
        tensors["q"], tensors["k"], tensors["v"], o, do, lse, k_self=tensors["k_self"],
        v_self=tensors["v_self"], **args)))
    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, t in tensors.items():
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in t.shape)
            old = t[idx]
            t[idx] = old + eps
            lp = loss(tensors)
            t[idx] = old - eps
            lm = loss(tensors)
            t[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


def test_bwd_zero_queries_closed_form_dv():
    """Q = 0, context only: P is uniform, so dV[j, g] = sum over queries that see j of
    sum over the group's heads of dO[i, h] / n_i."""
    meta, inp = tiny_case(4, self_block=False, chunk_size=70)
    q0 = np.zeros_like(inp.q.f64)
    o, lse = oracle.sparse_xattn_fwd(q0, inp.k.f64, inp.v.f64, meta.anchor, meta.sample_start,
                                     inp.chunk_gstart, inp.chunk_len, 1.0)
    _, _, dv, _, _ = oracle.sparse_xattn_bwd(q0, inp.k.f64, inp.v.f64, o, inp.dout.f64, lse,
                                             meta.anchor, meta.sample_start, inp.chunk_gstart,
                                             inp.chunk_len, 1.0)
    gpos = synth.chunk_rows(inp.chunk_gstart, inp.chunk_len)
    want = np.zeros_like(dv)
    for i in range(q0.shape[0]):
        b = i // 16
        sel = (meta.sample_start[b] <= gpos) & (gpos < meta.anchor[b])
        n = sel.sum()
        for h in range(4):
            want[sel, h // 2, :] += inp.dout.f64[i, h] / n
    np.testing.assert_allclose(dv, want, atol=1e-12)


# ----------------------------------------------------------------------------- cost

def test_cost_golden_tiny():
    g = json.load(open(os.path.join(GOLDEN, "cost_tiny.json")))
    c = oracle.chunk_cost(g["anchor"], g["sample_start"], g["n_ctx"], g["chunk_size"], g["block"])
    assert c.tolist() == g["cost"]


@pytest.mark.parametrize("seed", range(5))
def test_cost_closed_forms(seed):
    n_ctx = 700
    meta = synth.draw_meta(seed, n_ctx, 60, 300, 9)
    for cs in (1, 64, 100, 700, 1000):
        c = oracle.chunk_cost(meta.anchor, meta.sample_start, n_ctx, cs)
        assert c.dtype == np.int64 and len(c) == -(-n_ctx // cs)
        # total = 16 * sum over blocks of the interval length
        assert int(c.sum()) == 16 * int((meta.anchor.astype(np.int64) - meta.sample_start).sum())
    # unit chunks: cost[j] = 16 * #blocks whose interval contains j, by a difference array
    diff = np.zeros(n_ctx + 1, np.int64)
    np.add.at(diff, meta.sample_start, 16)
    np.add.at(diff, meta.anchor, -16)
    np.testing.assert_array_equal(oracle.chunk_cost(meta.anchor, meta.sample_start, n_ctx, 1),
                                  np.cumsum(diff)[:n_ctx])
    assert oracle.total_pairs(meta.anchor, meta.sample_start, n_ctx) == \
        16 * int((meta.anchor.astype(np.int64) - meta.sample_start).sum())


def test_cost_exceeds_int32_range_is_exact():
    """Costs are int64: a chunk read by many blocks can pass 2**31 at large sizes."""
    n_blk = 40000
    anchor = np.full(n_blk, 4096, np.int32)
    start = np.zeros(n_blk, np.int32)
    c = oracle.chunk_cost(anchor, start, 4096, 4096, chunks=[0])
    assert int(c[0]) == 16 * n_blk * 4096 and int(c[0]) > 2 ** 31


# ----------------------------------------------------------------------------- LPT

def test_lpt_golden():
    g = json.load(open(os.path.join(GOLDEN, "lpt_tiny.json")))
    for case in g["cases"]:
        b, load = oracle.lpt_assign(case["cost"], case["n_bin"])
        assert b == case["bin_of_chunk"] and load == case["bin_load"]


def test_imbalance_golden():
    """The work imbalance of a plan against hand-worked exact fractions (max / mean - 1).
    The values separate it from the plausible wrong readings: max / min - 1 gives 1/16
    on [17, 16] and is undefined on [8, 3, 3, 0]; (max - mean) / max gives 1/34."""
    from fractions import Fraction

    g = json.load(open(os.path.join(GOLDEN, "lpt_tiny.json")))
    cases = [(c["bin_load"], c["imbalance"]) for c in g["cases"]]
    cases += [(c["load"], c["imbalance"]) for c in g["imbalance_extra"]]
    assert len(cases) >= 7
    for load, want in cases:
        got = oracle.imbalance(load)
        assert abs(got - float(Fraction(want))) <= 1e-15, (load, got, want)


@pytest.mark.parametrize("seed", range(10))
def test_lpt_properties(seed):
    rng = np.random.default_rng(seed)
    n_bin = int(rng.integers(1, 9))
    n = n_bin * int(rng.integers(1, 9))
    cost = rng.integers(0, 50, size=n)
    bins, load = oracle.lpt_assign(cost, n_bin)
    counts = np.bincount(bins, minlength=n_bin)
    assert np.all(counts == n // n_bin)
    assert sum(load) == int(cost.sum())
    for p in range(n_bin):
        assert load[p] == int(cost[np.asarray(bins) == p].sum())


def test_lpt_special_cases():
    b, load = oracle.lpt_assign([7] * 12, 4)
    assert b == [i % 4 for i in range(12)]
    b, load = oracle.lpt_assign([3, 1, 4, 1, 5], 1)
    assert b == [0] * 5 and load == [14]
    with pytest.raises(ValueError):
        oracle.lpt_assign([1, 2, 3], 2)


def test_lpt_balances_a_generated_plan():
    """Sanity range, not a pin: on the 64k-context workload the plan is far better
    balanced than contiguous chunking (the pages report < 1 % imbalance on theirs)."""
    w = synth.WORKLOADS["fwd_bf16_8kq_64k"]
    meta = synth.meta_for(w, 3)
    cost = oracle.chunk_cost(meta.anchor, meta.sample_start, w.n_ctx, w.chunk_size)
    _, load = oracle.lpt_assign(cost, w.n_bin)
    contiguous = cost.reshape(w.n_bin, -1).sum(axis=1)
    assert oracle.imbalance(load) < 0.05
    assert oracle.imbalance(load) < oracle.imbalance(contiguous)
