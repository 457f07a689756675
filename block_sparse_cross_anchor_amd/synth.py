"""Seeded synthetic workloads for anchor-masked block-sparse cross-attention.

This module only *draws inputs*: packed sample lengths, anchor positions and
normally distributed tensors.  It holds none of the method's arithmetic (no
attention, no combine, no cost, no planning), so the CPU oracle and the GPU
path can both be fed from it without sharing any computation.

Shapes follow the Split-KV description of diffusion-drafter training
("Split-KV speeds diffusion drafter training...", section "Why short queries
change the problem"): anchors sampled inside each packed sample open blocks of
``BLOCK`` draft tokens; the query budget is ``n_anchor * BLOCK`` tokens and is
independent of the context length.

Random streams: every tensor kind has its own PCG64 stream keyed by
``SeedSequence([seed, tag, granule])``.  Context-side tensors (K, V) are drawn
in granules of ``GRANULE`` rows, so any subset of context rows (one device's
share of chunks) has exactly the values those rows have in the full context.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 16          # draft tokens per anchor block
GRANULE = 1024      # rows per independent K/V draw granule

# stream tags
_T_META, _T_Q, _T_K, _T_V, _T_KS, _T_VS, _T_DO, _T_PO, _T_PL = range(9)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: packed context, anchors, heads, dtype, chunking."""
    name: str
    n_ctx: int            # packed context length (tokens)
    len_lo: int           # sample length range, inclusive
    len_hi: int
    n_anchor: int         # anchors (= blocks); queries = n_anchor * BLOCK
    hq: int
    hkv: int
    d: int
    dtype: str            # "f32" or "bf16"
    value_std: str        # "unit": N(0,1); "inv_sqrt_d": N(0,1)/sqrt(d)
    chunk_size: int       # contiguous chunk length of the context partition
    n_bin: int = 0        # LPT bins (0: no planning step)
    bwd: bool = False     # workload includes the backward pass

    @property
    def n_q(self) -> int:
        return self.n_anchor * BLOCK

    @property
    def n_chunk(self) -> int:
        return -(-self.n_ctx // self.chunk_size)

    def std(self, d=None) -> float:
        d = self.d if d is None else d
        return 1.0 if self.value_std == "unit" else 1.0 / np.sqrt(d)


# The five workloads (tiny fp32 -> one device's share at CP size 64), plus the
# benchmark's forward+backward step on the 8192-query x 65536-token shapes.
WORKLOADS = {
    "tiny_fp32_512": Workload("tiny_fp32_512", 512, 512, 512, 4, 2, 2, 64, "f32", "unit", 256),
    "fwd_bf16_512q_4k": Workload("fwd_bf16_512q_4k", 4096, 512, 2048, 32, 32, 8, 128, "bf16",
                                 "inv_sqrt_d", 1024),
    "fwd_bf16_8kq_64k": Workload("fwd_bf16_8kq_64k", 65536, 4096, 32768, 512, 32, 8, 128, "bf16",
                                 "inv_sqrt_d", 1024, n_bin=8),
    # the same shapes and draws, forward and backward: the benchmark's step
    "fwdbwd_bf16_8kq_64k": Workload("fwdbwd_bf16_8kq_64k", 65536, 4096, 32768, 512, 32, 8, 128,
                                    "bf16", "inv_sqrt_d", 1024, n_bin=8, bwd=True),
    "fwdbwd_bf16_4kq_32k": Workload("fwdbwd_bf16_4kq_32k", 32768, 4096, 32768, 256, 32, 8, 128,
                                    "bf16", "inv_sqrt_d", 4096, bwd=True),
    "cp64_share_8kq_512k": Workload("cp64_share_8kq_512k", 524288, 8192, 65536, 512, 32, 8, 128,
                                    "bf16", "inv_sqrt_d", 1024, n_bin=64, bwd=True),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclass
class Meta:
    """Packed-context metadata.  Blocks are sorted by global anchor position."""
    lengths: np.ndarray        # int64 [n_sample]
    offsets: np.ndarray        # int64 [n_sample] start of each sample in the packed context
    anchor: np.ndarray         # int32 [n_blk] global position of each block's anchor
    sample_start: np.ndarray   # int32 [n_blk] global start of the block's sample
    n_ctx: int
    extra: dict = field(default_factory=dict)

    @property
    def n_blk(self) -> int:
        return int(self.anchor.shape[0])


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def draw_lengths(rng: np.random.Generator, n_ctx: int, lo: int, hi: int) -> np.ndarray:
    """Integer-uniform lengths in [lo, hi], packed until >= n_ctx, last one truncated."""
    out, total = [], 0
    while total < n_ctx:
        L = int(rng.integers(lo, hi, endpoint=True))
        out.append(L)
        total += L
    out[-1] -= total - n_ctx
    return np.asarray(out, dtype=np.int64)


def apportion(n: int, weights: np.ndarray) -> np.ndarray:
    """Largest-remainder apportionment of n items proportional to integer weights
    (exact integer arithmetic; ties on the remainder go to the lower index)."""
    w = np.asarray(weights, dtype=np.int64)
    tot = int(w.sum())
    num = n * w
    base = num // tot
    rem = num - base * tot
    left = n - int(base.sum())
    order = sorted(range(len(w)), key=lambda i: (-int(rem[i]), i))
    for i in order[:left]:
        base[i] += 1
    return base


def draw_meta(seed: int, n_ctx: int, len_lo: int, len_hi: int, n_anchor: int,
              block: int = BLOCK) -> Meta:
    """Sample lengths, then anchors: counts per sample proportional to length over
    samples of length >= 2*block; inside a sample, positions drawn uniformly without
    replacement from the relative range [block, L - block]; emitted sorted."""
    rng = _rng(seed, _T_META)
    lengths = draw_lengths(rng, n_ctx, len_lo, len_hi)
    offsets = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    elig = np.flatnonzero(lengths >= 2 * block)
    counts = np.zeros(len(lengths), dtype=np.int64)
    counts[elig] = apportion(n_anchor, lengths[elig])
    anchors, starts = [], []
    for s in range(len(lengths)):
        c = int(counts[s])
        if c == 0:
            continue
        L = int(lengths[s])
        avail = L - 2 * block + 1
        if c > avail:
            raise ValueError(f"sample {s} of length {L} cannot hold {c} anchors")
        rel = np.sort(rng.choice(np.arange(block, L - block + 1), size=c, replace=False))
        anchors.append(offsets[s] + rel)
        starts.append(np.full(c, offsets[s]))
    anchor = np.concatenate(anchors).astype(np.int32)
    sample_start = np.concatenate(starts).astype(np.int32)
    return Meta(lengths, offsets, anchor, sample_start, n_ctx)


def meta_for(w: Workload, seed: int) -> Meta:
    return draw_meta(seed, w.n_ctx, w.len_lo, w.len_hi, w.n_anchor)


# ----------------------------------------------------------------------------- tensors

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    # in 32-bit words: a finite value's bits plus at most 0x8000 stay below 2^32
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    odd = (u >> 16) & 1
    u += 0x7FFF
    u += odd
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """A drawn tensor: ``bits`` is what the device receives (float32 array, or uint16
    bf16 bit patterns); ``f64`` is the exact same values upcast to float64."""
    bits: np.ndarray
    dtype: str

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.bits).astype(np.float64)
        return self.bits.astype(np.float64)

    @property
    def shape(self):
        return self.bits.shape


def _finish(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x), "bf16")
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(x, dtype=np.float32), "f32")
    raise ValueError(dtype)


def draw_normal(seed: int, tag: int, shape, std: float, dtype: str, sub: int = 0) -> Tensor:
    rng = _rng(seed, tag, sub)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return _finish(x, dtype)


def draw_context(seed: int, tag: int, rows: np.ndarray, h: int, d: int, std: float,
                 dtype: str) -> Tensor:
    """Context tensor values at the given global rows (granule-wise streams).  Each
    granule's values are drawn, scaled and rounded on their own, so the output is
    built piecewise without whole-tensor temporaries."""
    rows = np.asarray(rows, dtype=np.int64)
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    out = np.empty((rows.shape[0], h, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    if rows.size:
        gran = rows // GRANULE
        order = np.argsort(gran, kind="stable")   # rows grouped by granule
        ug, first = np.unique(gran[order], return_index=True)
        ends = np.append(first[1:], order.size)
        for g, a, e in zip(ug, first, ends):
            rng = _rng(seed, tag, int(g))
            block = rng.standard_normal(size=(GRANULE, h, d), dtype=np.float32)
            if std != 1.0:
                block *= np.float32(std)
            sel = order[a:e]
            if sel[-1] - sel[0] == e - a - 1 and np.all(np.diff(sel) == 1):   # a run of rows
                sel = slice(int(sel[0]), int(sel[-1]) + 1)
            vals = block[rows[sel] - g * GRANULE]
            out[sel] = f32_to_bf16_bits(vals) if dtype == "bf16" else vals
    return Tensor(out, dtype)


def chunk_rows(chunk_gstart, chunk_len) -> np.ndarray:
    """Global rows of the local K/V buffer: the listed chunks back to back."""
    parts = [np.arange(int(s), int(s) + int(n)) for s, n in zip(chunk_gstart, chunk_len)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def contiguous_chunks(n_ctx: int, chunk_size: int):
    """The contiguous fixed-size partition of the packed context."""
    starts = np.arange(0, n_ctx, chunk_size, dtype=np.int32)
    lens = np.minimum(chunk_size, n_ctx - starts).astype(np.int32)
    return starts, lens


@dataclass
class Inputs:
    q: Tensor
    k: Tensor            # local rows (chunks back to back)
    v: Tensor
    k_self: Tensor | None
    v_self: Tensor | None
    dout: Tensor | None
    chunk_gstart: np.ndarray
    chunk_len: np.ndarray


def draw_inputs(seed: int, meta: Meta, hq: int, hkv: int, d: int, dtype: str, std: float,
                chunk_gstart, chunk_len, self_block: bool = True, with_dout: bool = False,
                dout_std: float = 1.0) -> Inputs:
    n_q = meta.n_blk * BLOCK
    q = draw_normal(seed, _T_Q, (n_q, hq, d), std, dtype)
    rows = chunk_rows(chunk_gstart, chunk_len)
    k = draw_context(seed, _T_K, rows, hkv, d, std, dtype)
    v = draw_context(seed, _T_V, rows, hkv, d, std, dtype)
    ks = vs = None
    if self_block:
        ks = draw_normal(seed, _T_KS, (n_q, hkv, d), std, dtype)
        vs = draw_normal(seed, _T_VS, (n_q, hkv, d), std, dtype)
    do = draw_normal(seed, _T_DO, (n_q, hq, d), dout_std, dtype) if with_dout else None
    return Inputs(q, k, v, ks, vs, do, np.asarray(chunk_gstart, np.int32),
                  np.asarray(chunk_len, np.int32))


def draw_partials(seed: int, n_parts: int, rows: int, d: int, dtype: str,
                  o_std: float = 0.1, lse_lo: float = 0.0, lse_hi: float = 10.0,
                  empty: np.ndarray | None = None):
    """Synthetic partial (O, lse) sets for the combine: lse ~ U(lse_lo, lse_hi),
    O ~ N(0, o_std^2).  ``empty`` [n_parts, rows] marks partials with no allowed key:
    those get lse = -inf and O = 0."""
    o = draw_normal(seed, _T_PO, (n_parts, rows, d), o_std, dtype)
    rng = _rng(seed, _T_PL)
    lse = rng.uniform(lse_lo, lse_hi, size=(n_parts, rows)).astype(np.float32)
    if empty is not None:
        empty = np.asarray(empty, dtype=bool)
        lse[empty] = -np.inf
        o.bits[empty] = 0
    return o, lse
