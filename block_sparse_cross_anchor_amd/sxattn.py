"""ctypes binding of libsxattn (C ABI in include/sxattn.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch tensors on the current HIP device (torch is used for
device memory and streams); each call is enqueued on torch's current stream.
The library must have been built (``python -m block_sparse_cross_anchor_amd.build``);
a missing library raises at the first call -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsxattn.so")

SXA_F32, SXA_BF16 = 0, 1
SXA_OK, SXA_EINVAL, SXA_EUNSUPPORTED, SXA_EHIP = 0, -1, -2, -3
BWD_DELTA, BWD_DQ, BWD_DKDV, BWD_DQ_OVERWRITE, BWD_DKDV_BF16 = 1, 2, 4, 8, 16
BLOCK = 16

EXPORTS = ("sparse_xattn_fwd", "sparse_xattn_fwd_noalloc", "sparse_xattn_fwd_workspace_bytes",
           "sparse_xattn_fwd_split_workspace_bytes", "sparse_xattn_bwd",
           "sparse_xattn_bwd_workspace_bytes", "sparse_xattn_bwd_split_workspace_bytes",
           "lse_combine", "chunk_cost", "lpt_assign", "lpt_plan", "context_gather", "sxa_last_error")

_lib = None


class SxaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sxattn status {status}: {message}")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libsxattn.so (or the build named by $SXATTN_LIB) and declare the prototypes
    of every exported entry point."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SXATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_cross_anchor_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    attn_common = [P, P, P, ctypes.c_int, I32, I32, I32, I32, I32, F32, P, P, P, P, I32, I64, P, P]
    lib.sparse_xattn_fwd.argtypes = attn_common + [P, ctypes.c_int, P, P, I64, P]
    lib.sparse_xattn_fwd.restype = ctypes.c_int
    lib.sparse_xattn_fwd_noalloc.argtypes = attn_common + [P, ctypes.c_int, P, P]
    lib.sparse_xattn_fwd_noalloc.restype = ctypes.c_int
    lib.sparse_xattn_fwd_workspace_bytes.argtypes = [I32, I32, I32]
    lib.sparse_xattn_fwd_workspace_bytes.restype = I64
    lib.sparse_xattn_fwd_split_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.sparse_xattn_fwd_split_workspace_bytes.restype = I64
    lib.sparse_xattn_bwd.argtypes = attn_common + [P, P, P, P, P, P, P, P, P, P, I64, I32, P]
    lib.sparse_xattn_bwd_workspace_bytes.argtypes = [I32, I64, I32, I32, I32]
    lib.sparse_xattn_bwd_workspace_bytes.restype = I64
    lib.sparse_xattn_bwd_split_workspace_bytes.argtypes = [I32, I64, I32, I32, I32]
    lib.sparse_xattn_bwd_split_workspace_bytes.restype = I64
    lib.sparse_xattn_bwd.restype = ctypes.c_int
    lib.lse_combine.argtypes = [P, ctypes.c_int, P, I32, I64, I32, P, ctypes.c_int, P, P]
    lib.lse_combine.restype = ctypes.c_int
    lib.chunk_cost.argtypes = [P, P, I32, I32, I32, I32, P, P]
    lib.chunk_cost.restype = ctypes.c_int
    lib.lpt_assign.argtypes = [P, I32, I32, P, P]
    lib.lpt_assign.restype = ctypes.c_int
    lib.lpt_plan.argtypes = [P, P, P, I32, I32, P, P, P, P, P]
    lib.lpt_plan.restype = ctypes.c_int
    lib.context_gather.argtypes = [P, I64, P, P, I32, I64, P, P]
    lib.context_gather.restype = ctypes.c_int
    lib.sxa_last_error.argtypes = []
    lib.sxa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != SXA_OK:
        msg = load_library().sxa_last_error().decode(errors="replace")
        raise SxaError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SXA_BF16
    if t.dtype == torch.float32:
        return SXA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


class Meta:
    """Device metadata of one attention call: per-block anchors and sample starts,
    and the local chunk list (int32 device tensors)."""

    def __init__(self, anchor, sample_start, chunk_gstart, chunk_len, n_loc=None, device="cuda"):
        def dev(x):
            return torch.as_tensor(x, dtype=torch.int32).to(device).contiguous()

        self.anchor = dev(anchor)
        self.sample_start = dev(sample_start)
        self.chunk_gstart = dev(chunk_gstart)
        self.chunk_len = dev(chunk_len)
        self.n_blk = int(self.anchor.numel())
        self.n_chunk = int(self.chunk_gstart.numel())
        self.n_loc = int(torch.as_tensor(chunk_len, dtype=torch.int64).sum()) if n_loc is None \
            else int(n_loc)


def sparse_xattn_fwd(q, k, v, meta: Meta, scale: float, k_self=None, v_self=None,
                     out_dtype=None, out=None, lse=None, workspace="auto"):
    """Partial forward over the local chunks (+ own-block term).  Returns (o, lse).
    ``workspace``: "auto" (cached scratch: heaviest row groups dispatched first),
    "split" (cached scratch of the split schedule: row groups with many key tiles
    also run as several merged pieces), None, or a device tensor."""
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q", dtype=q.dtype)
    _need(k, "k", (meta.n_loc, hkv, d), q.dtype)
    _need(v, "v", (meta.n_loc, hkv, d), q.dtype)
    if k_self is not None:
        _need(k_self, "k_self", (n_q, hkv, d), q.dtype)
        _need(v_self, "v_self", (n_q, hkv, d), q.dtype)
    if n_q != meta.n_blk * BLOCK:
        raise ValueError("q rows must equal 16 * number of blocks")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((n_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((n_q, hq), dtype=torch.float32, device=q.device)
    _need(out, "out", (n_q, hq, d), out_dtype)
    _need(lse, "lse", (n_q, hq), torch.float32)
    lib = load_library()
    if isinstance(workspace, str):
        if workspace not in ("auto", "split"):
            raise ValueError(f"workspace must be 'auto', 'split', None or a tensor, not {workspace!r}")
        with torch.cuda.device(q.device):
            ws_bytes = int(lib.sparse_xattn_fwd_split_workspace_bytes(meta.n_blk, hq, hkv, d)
                           if workspace == "split" else
                           lib.sparse_xattn_fwd_workspace_bytes(meta.n_blk, hq, hkv))
        workspace = _scratch("fwd_" + workspace, ws_bytes, q.device)
    else:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_xattn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), meta.n_blk, BLOCK, hq, hkv, d, float(scale),
        _ptr(meta.anchor), _ptr(meta.sample_start), _ptr(meta.chunk_gstart), _ptr(meta.chunk_len),
        meta.n_chunk, meta.n_loc, _ptr(k_self), _ptr(v_self), _ptr(out), _dtype_code(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream()))
    return out, lse


def sparse_xattn_fwd_noalloc(q, k, v, meta: Meta, scale: float, k_self=None, v_self=None,
                             out=None, lse=None):
    """sparse_xattn_fwd through the entry point that allocates nothing (its row-group
    ranking lives in a static device array of the library).  ``out`` and ``lse`` are
    required, so that the call itself allocates nothing either.  Returns (o, lse)."""
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q", dtype=q.dtype)
    _need(k, "k", (meta.n_loc, hkv, d), q.dtype)
    _need(v, "v", (meta.n_loc, hkv, d), q.dtype)
    if k_self is not None:
        _need(k_self, "k_self", (n_q, hkv, d), q.dtype)
        _need(v_self, "v_self", (n_q, hkv, d), q.dtype)
    if n_q != meta.n_blk * BLOCK:
        raise ValueError("q rows must equal 16 * number of blocks")
    if out is None or lse is None:
        raise ValueError("sparse_xattn_fwd_noalloc needs caller-allocated out and lse")
    _need(out, "out", (n_q, hq, d))
    _need(lse, "lse", (n_q, hq), torch.float32)
    _check(load_library().sparse_xattn_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), meta.n_blk, BLOCK, hq, hkv, d, float(scale),
        _ptr(meta.anchor), _ptr(meta.sample_start), _ptr(meta.chunk_gstart), _ptr(meta.chunk_len),
        meta.n_chunk, meta.n_loc, _ptr(k_self), _ptr(v_self), _ptr(out), _dtype_code(out),
        _ptr(lse), _stream()))
    return out, lse


_workspaces = {}


def _scratch(kind: str, need: int, device) -> torch.Tensor:
    """Cached device scratch per (kind, device, current stream), grown on demand.  Calls
    on one stream share it and are ordered by that stream; calls on different streams
    get different buffers, so they never race on it."""
    dev = torch.device(device)
    key = (kind, dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        # allocated on this stream: torch reuses a replaced buffer only in this
        # stream's order, after the work queued on it
        ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def bwd_workspace(n_blk: int, n_loc: int, hq: int, hkv: int, d: int, device, split=False):
    """Scratch of the load-balanced dQ and dK/dV phases (cached per device and stream), with the
    split dQ schedule's plan and slots when ``split``.  Returns (tensor, bytes to pass)."""
    lib = load_library()
    size = lib.sparse_xattn_bwd_split_workspace_bytes if split else lib.sparse_xattn_bwd_workspace_bytes
    with torch.cuda.device(torch.device(device)):
        need = int(size(int(n_blk), int(n_loc), int(hq), int(hkv), int(d)))
    return _scratch("bwd_split" if split else "bwd", need, device), need


def sparse_xattn_bwd(q, k, v, meta: Meta, scale: float, o, dout, lse, dq_accum,
                     k_self=None, v_self=None, delta_ws=None, dk=None, dv=None, dk_self=None,
                     dv_self=None, flags: int = 0, workspace="auto", grad_dtype=None):
    """Backward of the local chunks (+ own-block term).  Adds into dq_accum (float32)
    unless BWD_DQ_OVERWRITE is set; ``flags`` selects phases (none named = all).
    ``workspace``: "auto" (cached scratch: load-balanced phases), "split" (also the
    split dQ schedule), None, or a device tensor.  The key/value gradients are float32
    or bf16: the dtype of the given dk (``grad_dtype``, default float32, when dk is
    not given); bf16 sets BWD_DKDV_BF16.
    Returns the gradients (dk, dv, dk_self, dv_self)."""
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q")
    _need(k, "k", (meta.n_loc, hkv, d), q.dtype)
    _need(v, "v", (meta.n_loc, hkv, d), q.dtype)
    _need(o, "o", (n_q, hq, d), q.dtype)
    _need(dout, "dout", (n_q, hq, d), q.dtype)
    _need(lse, "lse", (n_q, hq), torch.float32)
    _need(dq_accum, "dq_accum", (n_q, hq, d), torch.float32)
    if delta_ws is None:
        delta_ws = torch.empty((2, n_q, hq), dtype=torch.float32, device=q.device)
    _need(delta_ws, "delta_ws", (2, n_q, hq), torch.float32)
    gd = dk.dtype if dk is not None else (grad_dtype or torch.float32)
    if gd not in (torch.float32, torch.bfloat16):
        raise TypeError(f"key/value gradients must be float32 or bfloat16, not {gd}")
    if dk is None:
        dk = torch.empty(k.shape, dtype=gd, device=k.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=gd, device=v.device)
    _need(dk, "dk", k.shape, gd)
    _need(dv, "dv", v.shape, gd)
    if k_self is not None:
        _need(k_self, "k_self", (n_q, hkv, d), q.dtype)
        _need(v_self, "v_self", (n_q, hkv, d), q.dtype)
        if dk_self is None:
            dk_self = torch.empty(k_self.shape, dtype=gd, device=q.device)
        if dv_self is None:
            dv_self = torch.empty(v_self.shape, dtype=gd, device=q.device)
        _need(dk_self, "dk_self", k_self.shape, gd)
        _need(dv_self, "dv_self", v_self.shape, gd)
    if gd == torch.bfloat16:
        flags = int(flags) | BWD_DKDV_BF16
    lib = load_library()
    if isinstance(workspace, str):
        if workspace not in ("auto", "split"):
            raise ValueError(f"workspace must be 'auto', 'split', None or a tensor, not {workspace!r}")
        workspace, ws_bytes = bwd_workspace(meta.n_blk, meta.n_loc, hq, hkv, d, q.device,
                                            split=workspace == "split")
    else:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_xattn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), meta.n_blk, BLOCK, hq, hkv, d, float(scale),
        _ptr(meta.anchor), _ptr(meta.sample_start), _ptr(meta.chunk_gstart), _ptr(meta.chunk_len),
        meta.n_chunk, meta.n_loc, _ptr(k_self), _ptr(v_self), _ptr(o), _ptr(dout), _ptr(lse),
        _ptr(delta_ws), _ptr(dq_accum), _ptr(dk), _ptr(dv), _ptr(dk_self), _ptr(dv_self),
        _ptr(workspace), ws_bytes, int(flags), _stream()))
    return dk, dv, dk_self, dv_self


def lse_combine(o_parts, lse_parts, out_dtype=None, out=None, lse_out=None):
    """o_parts [P, rows, d], lse_parts [P, rows] -> (o [rows, d], lse [rows])."""
    n_parts, rows, d = o_parts.shape
    _need(o_parts, "o_parts")
    _need(lse_parts, "lse_parts", (n_parts, rows), torch.float32)
    out_dtype = out_dtype or o_parts.dtype
    if out is None:
        out = torch.empty((rows, d), dtype=out_dtype, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    _need(out, "out", (rows, d), out_dtype)
    _need(lse_out, "lse_out", (rows,), torch.float32)
    lib = load_library()
    _check(lib.lse_combine(_ptr(o_parts), _dtype_code(o_parts), _ptr(lse_parts), n_parts, rows, d,
                           _ptr(out), _dtype_code(out), _ptr(lse_out), _stream()))
    return out, lse_out


def chunk_cost(anchor, sample_start, n_ctx: int, chunk_size: int, out=None):
    """int64 realised cost of every contiguous chunk (device tensor)."""
    _need(anchor, "anchor", dtype=torch.int32)
    _need(sample_start, "sample_start", anchor.shape, torch.int32)
    n_chunk = -(-int(n_ctx) // int(chunk_size)) if chunk_size > 0 else 0
    if out is None:
        out = torch.empty((max(n_chunk, 0),), dtype=torch.int64, device=anchor.device)
    lib = load_library()
    _check(lib.chunk_cost(_ptr(anchor), _ptr(sample_start), int(anchor.numel()), BLOCK, int(n_ctx),
                          int(chunk_size), _ptr(out), _stream()))
    return out


def context_gather(src, chunk_gstart, chunk_len, n_rows: int, out=None):
    """Rows of the listed chunks of ``src`` ([rows, ...] device tensor) back to back.
    chunk_gstart / chunk_len: int32 device tensors; n_rows = sum of the lengths."""
    _need(src, "src")
    _need(chunk_gstart, "chunk_gstart", dtype=torch.int32)
    _need(chunk_len, "chunk_len", chunk_gstart.shape, torch.int32)
    if out is None:
        out = torch.empty((int(n_rows),) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    _need(out, "out", (int(n_rows),) + tuple(src.shape[1:]), src.dtype)
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else 16
    lib = load_library()
    _check(lib.context_gather(_ptr(src), row_bytes, _ptr(chunk_gstart), _ptr(chunk_len),
                              int(chunk_gstart.numel()), int(n_rows), _ptr(out), _stream()))
    return out


def lpt_plan(cost, chunk_gstart, chunk_len, n_bin: int, bin_of=None, load=None, plan=None):
    """Device LPT plan, asynchronous on the current stream.  cost: int64, chunk_gstart
    and chunk_len: int32 CUDA tensors of n_chunk entries.  Returns (bin_of_chunk int32
    [n_chunk], bin_load int64 [n_bin], plan int32 [2, n_bin, n_chunk / n_bin]), plan[0]
    and plan[1] holding each bin's chunk starts and lengths in increasing chunk index."""
    n = int(cost.numel())
    nb = int(n_bin)
    for t, name, dt in ((cost, "cost", torch.int64), (chunk_gstart, "chunk_gstart", torch.int32),
                        (chunk_len, "chunk_len", torch.int32)):
        _need(t, name, (n,), dt)
    per = n // nb if nb > 0 else 0
    dev = cost.device
    bin_of = torch.empty((n,), dtype=torch.int32, device=dev) if bin_of is None else bin_of
    load = torch.empty((max(nb, 0),), dtype=torch.int64, device=dev) if load is None else load
    plan = torch.empty((2, max(nb, 0), per), dtype=torch.int32, device=dev) if plan is None else plan
    _need(bin_of, "bin_of", (n,), torch.int32)
    _need(load, "load", (max(nb, 0),), torch.int64)
    _need(plan, "plan", (2, max(nb, 0), per), torch.int32)
    _check(load_library().lpt_plan(_ptr(cost), _ptr(chunk_gstart), _ptr(chunk_len), n, nb, _ptr(bin_of),
                                   _ptr(load), _ptr(plan[0]), _ptr(plan[1]), _stream()))
    return bin_of, load, plan


def lpt_assign(cost, n_bin: int):
    """Host LPT plan.  cost: int64 CPU tensor/array.  Returns (bin_of_chunk, bin_load)."""
    c = torch.as_tensor(cost, dtype=torch.int64).contiguous()
    if c.is_cuda:
        raise ValueError("lpt_assign takes host costs")
    n = int(c.numel())
    bins = torch.empty((n,), dtype=torch.int32)
    load = torch.empty((max(int(n_bin), 0),), dtype=torch.int64)
    lib = load_library()
    _check(lib.lpt_assign(ctypes.c_void_p(c.data_ptr()), n, int(n_bin),
                          ctypes.c_void_p(bins.data_ptr()), ctypes.c_void_p(load.data_ptr())))
    return bins, load
