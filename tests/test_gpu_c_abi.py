"""The C ABI alone: a plain host program (tests/c_abi/sxattn_c_driver.cpp, built by
build()) calls chunk_cost, lpt_assign, sparse_xattn_fwd, lse_combine, context_gather
and sparse_xattn_bwd on HIP device buffers it allocates itself, with no Python or
PyTorch in the process.  Its outputs are compared with the oracle: costs and the plan
bit-exact, the gather bit-exact against slicing; the forward (with the own-block
term) and the two-call split merged by the combine at the bf16 tolerances; the
backward (from the driver's own forward; the oracle's from the oracle's forward) at
the gradient tolerance.
"""

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from block_sparse_cross_anchor_amd import synth
from helpers import assert_lse_close, rel_frob

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "sxattn_c_driver")


def bf16_f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("seed,order", [(2, "plain"), (21, "shuffled")])
def test_c_driver_matches_oracle(tmp_path, seed, order):
    if not os.path.exists(DRIVER):
        pytest.fail(f"{DRIVER} is missing: run build()")
    w = synth.WORKLOADS["fwd_bf16_512q_4k"]
    meta = synth.meta_for(w, seed)
    gs, gl = synth.contiguous_chunks(w.n_ctx, w.chunk_size)
    if order == "shuffled":   # chunks listed out of order, one of them split unevenly
        gs = np.array([3072, 1024, 0, 2048, 2560], np.int32)
        gl = np.array([1024, 1024, 1024, 512, 512], np.int32)
    inp = synth.draw_inputs(seed, meta, w.hq, w.hkv, w.d, "bf16", w.std(), gs, gl, with_dout=True)
    n_bin = 2
    d = tmp_path
    (d / "args.txt").write_text(f"{meta.n_blk} {w.hq} {w.hkv} {w.d} {w.n_ctx} {w.chunk_size} "
                                f"{n_bin} {len(gs)}\n")
    for name, arr in (("anchor", meta.anchor), ("start", meta.sample_start), ("gs", gs), ("gl", gl)):
        np.ascontiguousarray(arr, np.int32).tofile(d / f"{name}.bin")
    for name, t in (("q", inp.q), ("ks", inp.k_self), ("vs", inp.v_self), ("k", inp.k), ("v", inp.v),
                    ("dout", inp.dout)):
        np.ascontiguousarray(t.bits).tofile(d / f"{name}.bin")
    ggs, ggl = np.array([1500, 37], np.int32), np.array([700, 1000], np.int32)
    ggs.tofile(d / "ggs.bin")
    ggl.tofile(d / "ggl.bin")
    r = subprocess.run([DRIVER, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    cost = np.fromfile(d / "cost.bin", np.int64)
    want_cost = oracle.chunk_cost(meta.anchor, meta.sample_start, w.n_ctx, w.chunk_size)
    np.testing.assert_array_equal(cost, want_cost)
    want_bins, want_load = oracle.lpt_assign(want_cost, n_bin)
    assert np.fromfile(d / "bins.bin", np.int32).tolist() == want_bins
    assert np.fromfile(d / "load.bin", np.int64).tolist() == want_load
    # the device planner, from the device costs: the same plan, and each bin's chunks
    assert np.fromfile(d / "dbins.bin", np.int32).tolist() == want_bins
    assert np.fromfile(d / "dload.bin", np.int64).tolist() == want_load
    n_all = len(want_cost)
    all_gs = np.arange(n_all, dtype=np.int64) * w.chunk_size
    all_gl = np.minimum(w.chunk_size, w.n_ctx - all_gs)
    order = np.argsort(np.asarray(want_bins), kind="stable")
    np.testing.assert_array_equal(np.fromfile(d / "dplan_gs.bin", np.int32), all_gs[order])
    np.testing.assert_array_equal(np.fromfile(d / "dplan_gl.bin", np.int32), all_gl[order])

    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    ro, rl = oracle.sparse_xattn_fwd(inp.q.f64, inp.k.f64, inp.v.f64, meta.anchor,
                                     meta.sample_start, gs, gl, scale, inp.k_self.f64,
                                     inp.v_self.f64)
    for o_name, l_name in (("o", "lse"), ("o2", "lse2")):
        o = bf16_f64(np.fromfile(d / f"{o_name}.bin", np.uint16)).reshape(ro.shape)
        lse = np.fromfile(d / f"{l_name}.bin", np.float32).astype(np.float64).reshape(rl.shape)
        assert np.abs(o - ro).max() <= 2e-2 and rel_frob(o, ro) <= 1e-2, o_name
        assert_lse_close(lse, rl, 1e-3)

    kg = np.fromfile(d / "kg.bin", np.uint16).reshape(-1, w.hkv, w.d)
    kbits = np.ascontiguousarray(inp.k.bits)
    np.testing.assert_array_equal(kg, np.concatenate([kbits[1500:2200], kbits[37:1037]]))

    r = oracle.sparse_xattn_bwd(inp.q.f64, inp.k.f64, inp.v.f64, ro, inp.dout.f64, rl,
                                meta.anchor, meta.sample_start, gs, gl, scale, inp.k_self.f64,
                                inp.v_self.f64)
    for name, want in zip(("dq", "dk", "dv", "dks", "dvs"), r):
        got = np.fromfile(d / f"{name}.bin", np.float32).astype(np.float64).reshape(want.shape)
        assert rel_frob(got, want) <= 3e-2, name
