"""The device LPT plan (lpt_plan) against the oracle's LPT, bit for bit.

The plan is unique for given costs (chunks by cost descending then index, bins by
load then index), so the device's bin of every chunk and every bin's load must equal
the oracle's exactly; each bin's chunk list must be its chunks in increasing index.
Cases: random costs with many ties and zeros, loads far beyond 32 bits, one bin,
one chunk per bin, bins beyond one wave (lanes owning several bins), the size limits,
cost totals on both sides of 2^28 (up to 8 bins the greedy switches key width there),
and the benchmark workload's GPU-priced chunks.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import sxattn, synth

pytestmark = pytest.mark.gpu


def _check(cost_np, n_bin, gs=None, gl=None):
    n = len(cost_np)
    gs = np.arange(n, dtype=np.int32) * 7 + 3 if gs is None else gs
    gl = (np.arange(n, dtype=np.int32) % 5) + 1 if gl is None else gl
    cost = torch.as_tensor(np.asarray(cost_np, np.int64)).cuda()
    bin_of, load, plan = sxattn.lpt_plan(cost, torch.as_tensor(gs).cuda(), torch.as_tensor(gl).cuda(), n_bin)
    torch.cuda.synchronize()
    want_bins, want_load = oracle.lpt_assign([int(c) for c in cost_np], n_bin)
    want_bins = np.asarray(want_bins, np.int32)
    np.testing.assert_array_equal(bin_of.cpu().numpy(), want_bins)
    np.testing.assert_array_equal(load.cpu().numpy(), np.asarray(want_load, np.int64))
    order = np.argsort(want_bins, kind="stable").reshape(n_bin, n // n_bin)
    np.testing.assert_array_equal(plan[0].cpu().numpy(), gs[order])
    np.testing.assert_array_equal(plan[1].cpu().numpy(), gl[order])


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("seed", range(12))
def test_lpt_plan_random_costs_match_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    n_bin = int(rng.choice([1, 2, 3, 5, 8, 13, 64, 65, 100]))
    per = int(rng.integers(1, 9))
    pool = int(rng.choice([1, 3, 50, 10 ** 6]))   # few distinct values: many ties
    cost = rng.integers(0, pool, size=n_bin * per)
    _check(cost, n_bin)


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_lpt_plan_edge_cases():
    _check(np.zeros(64, np.int64), 8)                       # every cost equal
    _check(np.array([5], np.int64), 1)                       # one chunk, one bin
    _check(np.arange(16, dtype=np.int64)[::-1].copy(), 16)   # one chunk per bin
    big = np.array([2 ** 61, 2 ** 61 - 1, 3, 2 ** 60, 0, 2 ** 61, 7, 1], np.int64)
    _check(big, 2)                                           # loads beyond 32 bits (up to 2^62)
    rng = np.random.default_rng(7)
    _check(rng.integers(0, 1000, size=4096), 1024)           # the size limits
    _check(rng.integers(0, 10, size=4096), 8)
    # up to 8 bins, 32-bit keys hold the loads while the cost total stays below 2^28:
    # one case on each side of that switch, and one with a single cost past 2^63 / 4096
    for total in (2 ** 28 - 1, 2 ** 28):
        c = rng.integers(0, 2 ** 17, size=200 * 8).astype(np.int64)
        c[0] += total - int(c.sum())
        assert c.min() >= 0 and int(c.sum()) == total
        _check(c, 8)
        _check(c, 5)
    c = rng.integers(0, 3, size=64).astype(np.int64)
    c[5] = 2 ** 62
    _check(c, 8)


@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("name,n_bin", [("fwdbwd_bf16_8kq_64k", 8), ("cp64_share_8kq_512k", 64)])
def test_lpt_plan_on_gpu_priced_chunks(name, n_bin):
    """The step's own path: chunk_cost on the GPU, then lpt_plan on the GPU."""
    w = synth.WORKLOADS[name]
    meta = synth.meta_for(w, 3)
    anchor = torch.as_tensor(meta.anchor).cuda()
    start = torch.as_tensor(meta.sample_start).cuda()
    cost = sxattn.chunk_cost(anchor, start, w.n_ctx, w.chunk_size)
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    bin_of, load, plan = sxattn.lpt_plan(cost, torch.as_tensor(gs).cuda(), torch.as_tensor(gl).cuda(), n_bin)
    torch.cuda.synchronize()
    want_cost = oracle.chunk_cost(meta.anchor, meta.sample_start, w.n_ctx, w.chunk_size)
    want_bins, want_load = oracle.lpt_assign(want_cost, n_bin)
    np.testing.assert_array_equal(bin_of.cpu().numpy(), np.asarray(want_bins, np.int32))
    np.testing.assert_array_equal(load.cpu().numpy(), np.asarray(want_load, np.int64))
    order = np.argsort(np.asarray(want_bins), kind="stable").reshape(n_bin, -1)
    np.testing.assert_array_equal(plan[0].cpu().numpy(), gs[order])
    np.testing.assert_array_equal(plan[1].cpu().numpy(), gl[order])
