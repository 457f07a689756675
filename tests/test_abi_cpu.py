"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every
entry point declared in include/sxattn.h, rejects bad arguments before touching
the device, and its host LPT planner is bit-identical to the oracle's."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from block_sparse_cross_anchor_amd import sxattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sxattn.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sxattn.LIB_PATH):
        pytest.skip("libsxattn.so not built")
    return sxattn.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_symbols() == sorted(sxattn.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_invalid_arguments_are_rejected_on_the_host(lib):
    null = None
    # block size other than 16
    st_ = lib.chunk_cost(null, null, 1, 8, 100, 10, null, null)
    assert st_ == sxattn.SXA_EUNSUPPORTED
    assert b"block_size" in lib.sxa_last_error()
    # chunk size 0
    assert lib.chunk_cost(null, null, 0, 16, 100, 0, null, null) == sxattn.SXA_EINVAL
    # LPT: counts not divisible
    cost = (ctypes.c_int64 * 3)(1, 2, 3)
    bins = (ctypes.c_int32 * 3)()
    load = (ctypes.c_int64 * 2)()
    assert lib.lpt_assign(cost, 3, 2, bins, load) == sxattn.SXA_EINVAL
    # device LPT: counts not divisible, no bin, beyond its one-workgroup sizes, NULL
    # pointers (all rejected before anything is launched)
    fake = ctypes.c_void_p(16)
    plan_args = [fake] * 3 + [3, 2] + [fake] * 4 + [null]
    assert lib.lpt_plan(*plan_args) == sxattn.SXA_EINVAL
    plan_args[3], plan_args[4] = 4, 0
    assert lib.lpt_plan(*plan_args) == sxattn.SXA_EINVAL
    plan_args[3], plan_args[4] = 8192, 8
    assert lib.lpt_plan(*plan_args) == sxattn.SXA_EUNSUPPORTED
    assert b"4096" in lib.sxa_last_error()
    plan_args[3], plan_args[4] = 4096, 2048
    assert lib.lpt_plan(*plan_args) == sxattn.SXA_EUNSUPPORTED
    plan_args[3], plan_args[4], plan_args[5] = 64, 8, null
    assert lib.lpt_plan(*plan_args) == sxattn.SXA_EINVAL
    # attention: head_dim 96 unsupported, hq not a multiple of hkv, bad scale
    args = [null, null, null, 1, 1, 16, 4, 2, 96, 0.1, null, null, null, null, 0, 0, null, null,
            null, 1, null, null, 0, null]
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EUNSUPPORTED
    args[8], args[6], args[7] = 128, 6, 4
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EINVAL
    args[6], args[7], args[9] = 4, 2, -1.0
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EINVAL
    # float32 in, bf16 out
    args[9], args[19] = 0.1, sxattn.SXA_BF16
    args[3], args[4] = sxattn.SXA_F32, 0
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EUNSUPPORTED
    # size limits: more than 4096 kv heads, 2^29 or more query rows
    args[3], args[19] = sxattn.SXA_BF16, sxattn.SXA_BF16
    args[6], args[7] = 8192, 8192
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EUNSUPPORTED
    assert b"hkv" in lib.sxa_last_error()
    args[6], args[7], args[4] = 4, 2, 1 << 23  # 2^23 blocks x 16 x 4 heads = 2^29 rows
    assert lib.sparse_xattn_fwd(*args) == sxattn.SXA_EUNSUPPORTED
    assert b"2^29" in lib.sxa_last_error()
    args[4] = 1
    # combine: unsupported d
    assert lib.lse_combine(null, 1, null, 1, 10, 96, null, 1, null, null) == sxattn.SXA_EUNSUPPORTED
    # a good call clears the message
    assert lib.lpt_assign((ctypes.c_int64 * 2)(1, 2), 2, 2, (ctypes.c_int32 * 2)(),
                          (ctypes.c_int64 * 2)()) == sxattn.SXA_OK
    assert lib.sxa_last_error() == b""


def test_lpt_golden(lib):
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "lpt_tiny.json")))
    for case in g["cases"]:
        bins, load = sxattn.lpt_assign(np.asarray(case["cost"], np.int64), case["n_bin"])
        assert bins.tolist() == case["bin_of_chunk"] and load.tolist() == case["bin_load"]


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 16), st.integers(1, 12),
       st.lists(st.integers(0, 40), min_size=1, max_size=400), st.booleans())
def test_lpt_matches_oracle_bit_exact(lib, n_bin, per_bin, pool, wide):
    n = n_bin * per_bin
    cost = np.resize(np.asarray(pool, np.int64), n)
    if wide:
        cost = cost * np.int64(3_000_000_007)  # beyond int32
    want_bins, want_load = oracle.lpt_assign(cost, n_bin)
    bins, load = sxattn.lpt_assign(cost, n_bin)
    assert bins.tolist() == want_bins
    assert load.tolist() == want_load


def test_workspace_size_queries(lib):
    """Sizes of the optional workspaces: 0 for invalid sizes; the split schedule's
    scratch holds the job list, the split-group list and float32 slots for at most
    2 n_cu / hkv pieces of 256 rows (n_cu: the device's compute units, 256 where no
    device answers); the backward's split size is its plain size rounded up to 256
    plus the same scratch."""
    import torch
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    up = lambda x: -(-x // 256) * 256
    assert lib.sparse_xattn_fwd_split_workspace_bytes(512, 32, 8, 96) == 0
    assert lib.sparse_xattn_fwd_split_workspace_bytes(512, 30, 8, 128) == 0
    assert lib.sparse_xattn_fwd_split_workspace_bytes(-1, 32, 8, 128) == 0
    assert lib.sparse_xattn_fwd_split_workspace_bytes(0, 32, 8, 128) == 0        # no row group
    assert lib.sparse_xattn_fwd_split_workspace_bytes(4096 * 4 + 1, 32, 8, 128) == 0  # > 4096 groups
    assert lib.sparse_xattn_bwd_split_workspace_bytes(512, 65536, 32, 8, 96) == 0
    for n_blk, hq, hkv, d in ((512, 32, 8, 128), (40, 40, 1, 64), (3, 12, 4, 128)):
        split = lib.sparse_xattn_fwd_split_workspace_bytes(n_blk, hq, hkv, d)
        groups = -(-n_blk * 16 * (hq // hkv) // 256)
        assert lib.sparse_xattn_fwd_workspace_bytes(n_blk, hq, hkv) == 4 * groups
        pieces = max(2, -(-2 * n_cu // hkv))
        assert split == (up(16 * (groups + pieces)) + up(16 * (pieces // 2))
                         + up(4 * pieces * hkv * 256) + 4 * pieces * hkv * 256 * d)
        n_loc = 8192
        bwd = lib.sparse_xattn_bwd_workspace_bytes(n_blk, n_loc, hq, hkv, d)
        assert lib.sparse_xattn_bwd_split_workspace_bytes(n_blk, n_loc, hq, hkv, d) == up(bwd) + split
