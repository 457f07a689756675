"""Host-side helpers: the seeded input generator and the balance study's tile counts.

The generator feeds both the oracle and the GPU path, so its context draw must give
a row the same value whichever subset of rows is drawn (a device's share holds
exactly the full context's values), and its bf16 rounding must be round-to-nearest-
even.  The balance study's per-chunk tile counts are checked against an explicit
enumeration of tiles.
"""

import numpy as np
import pytest

import bench
from block_sparse_cross_anchor_amd import synth


def test_context_rows_do_not_depend_on_the_subset_drawn():
    full = synth.draw_context(11, 2, np.arange(3 * synth.GRANULE + 100), 2, 8, 0.5, "bf16").bits
    rng = np.random.default_rng(0)
    for rows in (rng.integers(0, full.shape[0], 700),                 # random, repeats
                 np.arange(synth.GRANULE - 5, 2 * synth.GRANULE + 7),  # a run across granules
                 np.array([3 * synth.GRANULE + 99, 0, 5])):            # unsorted
        sub = synth.draw_context(11, 2, rows, 2, 8, 0.5, "bf16").bits
        assert sub.dtype == np.uint16 and (sub == full[rows]).all()
    f32 = synth.draw_context(11, 2, np.arange(50), 2, 8, 0.5, "f32").bits
    assert f32.dtype == np.float32
    assert (synth.f32_to_bf16_bits(f32) == full[:50]).all()
    assert synth.draw_context(11, 2, np.zeros(0, np.int64), 2, 8, 1.0, "bf16").bits.shape == (0, 2, 8)


def test_bf16_rounding_is_nearest_even():
    # (float32 bits, expected bf16 bits)
    cases = [(0x3F800000, 0x3F80),   # 1.0 exact
             (0x3F808000, 0x3F80),   # tie, even stays
             (0x3F818000, 0x3F82),   # tie, odd rounds up
             (0x3F808001, 0x3F81),   # above the tie
             (0x3F807FFF, 0x3F80),   # below the tie
             (0xBF818000, 0xBF82),   # negative tie
             (0x7F7FFFFF, 0x7F80),   # largest finite rounds to inf (nearest even)
             (0x00000001, 0x0000),   # smallest subnormal
             (0x80000000, 0x8000)]   # -0
    x = np.array([c[0] for c in cases], np.uint32).view(np.float32)
    got = synth.f32_to_bf16_bits(x)
    assert got.tolist() == [c[1] for c in cases]
    # exhaustively over the low 16 bits of one exponent band, against integer arithmetic
    u = (np.uint32(0x40490000) + np.arange(1 << 16, dtype=np.uint32))
    ref = (u >> 16) + (((u & 0xFFFF) > 0x8000) | (((u & 0xFFFF) == 0x8000) & ((u >> 16) & 1 == 1)))
    assert (synth.f32_to_bf16_bits(u.view(np.float32)) == ref.astype(np.uint16)).all()


def _tiles_brute(groups, cs, ce, tk):
    out = np.zeros(len(cs), np.int64)
    for c in range(len(cs)):
        for lo, hi in groups:
            for t0 in range(cs[c], ce[c], tk):
                if max(lo, t0) < min(hi, min(t0 + tk, ce[c])):
                    out[c] += 1
    return out


@pytest.mark.parametrize("workload,seed", [("fwd_bf16_512q_4k", 2), ("tiny_fp32_512", 1)])
def test_balance_tile_costs_match_enumeration(workload, seed):
    w = synth.WORKLOADS[workload]
    meta = synth.meta_for(w, seed)
    tc, gt = bench.tile_costs(meta, w.n_ctx, w.chunk_size, w.hq, w.hkv)
    cs = np.arange(0, w.n_ctx, w.chunk_size)
    ce = np.minimum(cs + w.chunk_size, w.n_ctx)
    blk = list(zip(meta.sample_start.tolist(), meta.anchor.tolist()))
    tok = 256 // (w.hq // w.hkv)
    bpg = max(tok // 16, 1)
    grp = [(min(s for s, _ in blk[i:i + bpg]), max(a for _, a in blk[i:i + bpg]))
           for i in range(0, len(blk), bpg)]
    assert (tc["fwd_tiles"] == tok * 64 * _tiles_brute(grp, cs, ce, 64)).all()
    assert (tc["blk_tiles"] == 16 * 64 * _tiles_brute(blk, cs, ce, 64)).all()
    assert (tc["dkdv_tiles"] == 16 * 256 * _tiles_brute(blk, cs, ce, 256)).all()
    assert gt.shape == (len(grp), len(cs)) and (tok * 64 * gt.sum(0) == tc["fwd_tiles"]).all()
    # whole tiles cover at least the allowed pairs of each chunk
    lo = meta.sample_start.astype(np.int64)[:, None]
    hi = meta.anchor.astype(np.int64)[:, None]
    pairs = (16 * np.clip(np.minimum(hi, ce) - np.maximum(lo, cs), 0, None)).sum(0)
    for v in tc.values():
        assert (v >= pairs).all()


def test_dispatch_makespan():
    # equal jobs: rounds of n_cu; one long job bounds the makespan from below
    assert bench.dispatch_makespan([4] * 10, 5, 1) == 10
    assert bench.dispatch_makespan([20, 1, 1, 1], 4, 0) == 20
    assert bench.dispatch_makespan([3, 3, 2, 2, 2], 2, 0) == 7   # greedy, longest first (the optimum is 6)



def test_split_jobs():
    # jobs at or under the cap stay whole; a longer one becomes equal pieces, each
    # paying the merge
    assert bench.split_jobs([4, 8], 8, 1) == [4, 8]
    assert bench.split_jobs([20], 8, 1) == pytest.approx([20 / 3 + 1] * 3)
    # one long job on many units: splitting shortens the makespan
    assert bench.dispatch_makespan(bench.split_jobs([20, 1, 1, 1], 5, 1), 8, 0) == 6
    # every unit already busy: the merges only add work
    jobs = [10] * 16
    assert bench.dispatch_makespan(bench.split_jobs(jobs, 5, 1), 8, 2) > bench.dispatch_makespan(jobs, 8, 2)


def test_line_fit():
    x = np.array([1.0, 2.0, 3.0, 5.0])
    r2, worst = bench._fit(x, 2.0 + 3.0 * x)
    assert r2 == pytest.approx(1.0) and worst < 1e-12
    r2, _ = bench._fit(x, np.array([1.0, 3.0, 2.0, 4.0]))
    assert 0.0 < r2 < 1.0
