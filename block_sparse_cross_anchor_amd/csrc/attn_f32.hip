// Float32 path of the anchor-masked block-sparse cross-attention (forward and
// backward), plus the delta = rowsum(dO * O) pre-pass shared with the bf16 path.
//
// Mask ("Split-KV speeds diffusion drafter training...", section "Why short
// queries change the problem"): block b's 16 queries attend to the context
// positions [sample_start[b], anchor[b]) that lie in this call's chunks, plus the
// 16 own-block keys (rows 16b..16b+15 of k_self/v_self).  Partials carry the
// natural-log log-sum-exp so that they merge exactly (section "Exchange the
// smaller side").
//
// One workgroup per (block, head) walks the block's allowed key ranges in tiles of
// 64; the products run on gfx950's float32 matrix cores (v_mfma_f32_16x16x4_f32:
// float32 products and sums, so the float32 bound holds), the softmax on the VALU.
// The backward recomputes probabilities from the merged lse: P = exp(s - lse),
// dS = P (dO.V - delta), dQ += scale dS K (query-major kernel), dK = scale dS^T Q,
// dV = P^T dO summed over the group's heads (key-major kernel).
#include "device_common.h"
#include "internal.h"

namespace sxa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

// Walks the local rows of block b's allowed context keys: for every chunk, the
// intersection of [lo, hi) with the chunk, split into tiles of at most kTile rows.
template <typename F>
__device__ void for_each_ctx_tile(const AttnArgs& a, int lo, int hi, F&& f) {
  int64_t off = 0;
  for (int c = 0; c < a.n_chunk; ++c) {
    const int gs = a.chunk_gstart[c], len = a.chunk_len[c];
    const int s = max(lo, gs), e = min(hi, gs + len);
    if (s < e) {
      for (int64_t r = off + (s - gs); r < off + (e - gs); r += kTile)
        f(r, static_cast<int>(min<int64_t>(kTile, off + (e - gs) - r)));
    }
    off += len;
  }
}

// One float32 matrix-core product step, D += A B with A 16x4, B 4x16 (lane l gives
// A[l % 16][l / 16] and B[l / 16][l % 16]; it holds D[4 (l / 16) + r][l % 16] in r).
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Forward: one workgroup (4 waves) per (block, head), the block's allowed keys in
// tiles of 64 staged in LDS.  Per tile, wave w forms S^T = K Q^T for keys
// [16 w, 16 w + 16) on the matrix cores; the online softmax runs on the VALU, 16
// threads per query row; then O^T += V^T P^T on the matrix cores, each wave owning
// D / 64 of the 16-column tiles of O^T (so a lane's accumulators are one query's).
template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(AttnArgs a) {
  constexpr int TPW = D / 64;  // 16-column tiles of O^T per wave
  const int b = blockIdx.x, h = blockIdx.y;
  const int g = h / (a.hq / a.hkv);
  const int lo = a.sample_start[b], hi = a.anchor[b];
  const float* Q = static_cast<const float*>(a.q);
  __shared__ float qs[kBlock][D + 1];
  __shared__ float ks[kTile][D + 1];
  __shared__ float vs[kTile][D + 1];
  __shared__ float ps[kBlock][kTile + 1];  // scores, then probabilities
  __shared__ float alpha_s[kBlock], l_s[kBlock];
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l16 = lane % 16, q4 = lane / 16;
  for (int idx = tid; idx < kBlock * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    qs[i][c] = Q[(static_cast<int64_t>(kBlock * b + i) * a.hq + h) * D + c];
  }
  const int row = tid / 16, cg = tid % 16;  // softmax: 16 threads per query row
  float m = -INFINITY, l = 0.f;
  f32x4 oacc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const float* K, const float* V, int64_t row0, int nrows) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kThreads) {
      const int j = idx / D, c = idx % D;
      const int64_t src = ((row0 + j) * a.hkv + g) * D + c;
      ks[j][c] = j < nrows ? K[src] : 0.f;  // rows past the tile: finite, masked below
      vs[j][c] = j < nrows ? V[src] : 0.f;
    }
    __syncthreads();
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kk = 0; kk < D / 4; ++kk) sc = mma4(ks[16 * wave + l16][4 * kk + q4], qs[l16][4 * kk + q4], sc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * wave + 4 * q4 + r;
      ps[l16][key] = key < nrows ? sc[r] * a.scale : -INFINITY;
    }
    __syncthreads();
    float x[kTile / 16], tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTile / 16; ++u) {
      x[u] = ps[row][cg + 16 * u];
      tmax = fmaxf(tmax, x[u]);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 16));
    const float mnew = fmaxf(m, tmax);
    const float alpha = m == -INFINITY ? 0.f : expf(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < kTile / 16; ++u) {
      const int j = cg + 16 * u;
      const float pv = j < nrows ? expf(x[u] - mnew) : 0.f;
      ps[row][j] = pv;
      rs += pv;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) rs += __shfl_xor(rs, off, 16);
    l = l * alpha + rs;
    m = mnew;
    if (cg == 0) alpha_s[row] = alpha;
    __syncthreads();
    const float al = alpha_s[l16];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int dt = wave + 4 * t;
      oacc[t] *= al;
#pragma unroll 4
      for (int kk = 0; kk < kTile / 4; ++kk)
        oacc[t] = mma4(vs[4 * kk + q4][16 * dt + l16], ps[l16][4 * kk + q4], oacc[t]);
    }
  };

  if (a.k_self != nullptr)
    process(static_cast<const float*>(a.k_self), static_cast<const float*>(a.v_self),
            static_cast<int64_t>(kBlock) * b, kBlock);
  for_each_ctx_tile(a, lo, hi, [&](int64_t r0, int n) {
    process(static_cast<const float*>(a.k), static_cast<const float*>(a.v), r0, n);
  });

  if (cg == 0) {
    l_s[row] = l;
    const int64_t orow = static_cast<int64_t>(kBlock * b + row) * a.hq + h;
    a.lse[orow] = l > 0.f ? m + logf(l) : -INFINITY;
  }
  __syncthreads();
  const float lq = l_s[l16];
  const float inv = lq > 0.f ? 1.f / lq : 0.f;
  const int64_t orow = static_cast<int64_t>(kBlock * b + l16) * a.hq + h;
  float* O = static_cast<float*>(a.o);
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[orow * D + 16 * (wave + 4 * t) + 4 * q4 + r] = oacc[t][r] * inv;
}

// delta[row] = sum_d dout[row][d] * o[row][d], and delta[rows + row] = lse[row] in
// log2 units (the per-row inputs of the bf16 backward); 16 lanes per row.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(const T* __restrict__ o,
                                                         const T* __restrict__ dout,
                                                         const float* __restrict__ lse,
                                                         float* __restrict__ delta, int64_t rows) {
  constexpr int EPL = D / 16;
  const int lane = threadIdx.x % 16;
  const int64_t r_raw = static_cast<int64_t>(blockIdx.x) * (kThreads / 16) + threadIdx.x / 16;
  const int64_t r = r_raw < rows ? r_raw : rows - 1;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int64_t idx = r * D + lane * EPL + i;
    s = fmaf(load_as_f32<T>(dout + idx), load_as_f32<T>(o + idx), s);
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off, 16);
  if (lane == 0 && r_raw < rows) {
    delta[r] = s;
    // second plane: lse in log2 units, +inf for rows without any key (exp2(x - inf) = 0)
    const float l = lse[r];
    delta[rows + r] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// Query-major backward: dq_accum[i][h] += scale * sum_j dS_ij K_j over this call's keys.
// Per 64-key tile, wave w forms S^T = K Q^T and dP^T = V dO^T for keys [16 w, 16 w + 16)
// on the matrix cores and dS = P (dP - delta) in place; then dQ^T += K^T dS^T, each
// wave owning D / 64 of the 16-column tiles.
template <int D>
__global__ __launch_bounds__(kThreads) void dq_f32_kernel(AttnArgs a, bool overwrite) {
  constexpr int TPW = D / 64;
  const int b = blockIdx.x, h = blockIdx.y;
  const int g = h / (a.hq / a.hkv);
  const int lo = a.sample_start[b], hi = a.anchor[b];
  const float* Q = static_cast<const float*>(a.q);
  const float* dO = static_cast<const float*>(a.dout);
  __shared__ float qs[kBlock][D + 1];
  __shared__ float dos[kBlock][D + 1];
  __shared__ float ks[kTile][D + 1];
  __shared__ float vs[kTile][D + 1];
  __shared__ float dss[kBlock][kTile + 1];
  __shared__ float lse_s[kBlock], del_s[kBlock];
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l16 = lane % 16, q4 = lane / 16;
  for (int idx = tid; idx < kBlock * D; idx += kThreads) {
    const int i = idx / D, c = idx % D;
    const int64_t src = (static_cast<int64_t>(kBlock * b + i) * a.hq + h) * D + c;
    qs[i][c] = Q[src];
    dos[i][c] = dO[src];
  }
  if (tid < kBlock) {
    const int64_t r = static_cast<int64_t>(kBlock * b + tid) * a.hq + h;
    lse_s[tid] = a.lse_in[r];
    del_s[tid] = a.delta[r];
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const float* K, const float* V, int64_t row0, int nrows) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kThreads) {
      const int j = idx / D, c = idx % D;
      const int64_t src = ((row0 + j) * a.hkv + g) * D + c;
      ks[j][c] = j < nrows ? K[src] : 0.f;
      vs[j][c] = j < nrows ? V[src] : 0.f;
    }
    __syncthreads();
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kk = 0; kk < D / 4; ++kk) {
      sc = mma4(ks[16 * wave + l16][4 * kk + q4], qs[l16][4 * kk + q4], sc);
      dp = mma4(vs[16 * wave + l16][4 * kk + q4], dos[l16][4 * kk + q4], dp);
    }
    const float lq = lse_s[l16], dq_ = del_s[l16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * wave + 4 * q4 + r;
      float ds = 0.f;
      if (key < nrows && lq != -INFINITY) ds = expf(sc[r] * a.scale - lq) * (dp[r] - dq_);
      dss[l16][key] = ds;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int dt = wave + 4 * t;
#pragma unroll 4
      for (int kk = 0; kk < kTile / 4; ++kk)
        acc[t] = mma4(ks[4 * kk + q4][16 * dt + l16], dss[l16][4 * kk + q4], acc[t]);
    }
  };

  if (a.k_self != nullptr)
    process(static_cast<const float*>(a.k_self), static_cast<const float*>(a.v_self),
            static_cast<int64_t>(kBlock) * b, kBlock);
  for_each_ctx_tile(a, lo, hi, [&](int64_t r0, int n) {
    process(static_cast<const float*>(a.k), static_cast<const float*>(a.v), r0, n);
  });
  const int64_t orow = static_cast<int64_t>(kBlock * b + l16) * a.hq + h;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = a.dq + orow * D + 16 * (wave + 4 * t) + 4 * q4 + r;
      *dst = overwrite ? a.scale * acc[t][r] : *dst + a.scale * acc[t][r];
    }
}

// Key-major backward over tiles of 16 key rows: the local context rows, then (when
// k_self is given) one tile per block of own-block rows.  dK, dV are overwritten.
// Per (block, head) that may read the tile: wave 0 forms S^T = K Q^T and dP^T = V dO^T
// (16 keys x 16 queries) on the matrix cores and writes P and dS; then every wave adds
// dV^T += dO^T P and dK^T += Q^T dS for its D / 64 of the 16-column tiles.
template <int D>
__global__ __launch_bounds__(kThreads) void dkdv_f32_kernel(AttnArgs a, int n_ctx_tiles) {
  constexpr int TPW = D / 64;
  const int kt = blockIdx.x, g = blockIdx.y;
  const int grp = a.hq / a.hkv;
  const bool self_tile = kt >= n_ctx_tiles;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, l16 = lane % 16, q4 = lane / 16;
  const float* K = static_cast<const float*>(self_tile ? a.k_self : a.k);
  const float* V = static_cast<const float*>(self_tile ? a.v_self : a.v);
  const float* Q = static_cast<const float*>(a.q);
  const float* dO = static_cast<const float*>(a.dout);
  __shared__ float ks[kBlock][D + 1];
  __shared__ float vs[kBlock][D + 1];
  __shared__ float qs[kBlock][D + 1];
  __shared__ float dos[kBlock][D + 1];
  __shared__ float ps[kBlock][kBlock + 1];   // [query][key]
  __shared__ float dss[kBlock][kBlock + 1];  // [query][key]
  __shared__ int gpos[kBlock];
  __shared__ float lse_s[kBlock], del_s[kBlock];
  const int64_t row0 = self_tile ? static_cast<int64_t>(kt - n_ctx_tiles) * kBlock
                                 : static_cast<int64_t>(kt) * kBlock;
  const int64_t row_end = self_tile ? row0 + kBlock : min<int64_t>(row0 + kBlock, a.n_loc);
  const int nrows = static_cast<int>(row_end - row0);
  if (tid < kBlock) {
    int gp = -1;
    if (!self_tile && tid < nrows) {
      const int64_t r = row0 + tid;
      int64_t off = 0;
      for (int c = 0; c < a.n_chunk; ++c) {
        const int len = a.chunk_len[c];
        if (r >= off && r < off + len) {
          gp = a.chunk_gstart[c] + static_cast<int>(r - off);
          break;
        }
        off += len;
      }
    }
    gpos[tid] = gp;
  }
  for (int idx = tid; idx < kBlock * D; idx += kThreads) {
    const int j = idx / D, c = idx % D;
    float kv = 0.f, vv = 0.f;
    if (j < nrows) {
      const int64_t src = ((row0 + j) * a.hkv + g) * D + c;
      kv = K[src];
      vv = V[src];
    }
    ks[j][c] = kv;
    vs[j][c] = vv;
  }
  __syncthreads();
  f32x4 dk[TPW], dv[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) dk[t] = dv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int b_begin = self_tile ? kt - n_ctx_tiles : 0;
  const int b_end = self_tile ? b_begin + 1 : a.n_blk;
  for (int b = b_begin; b < b_end; ++b) {
    const int lo = a.sample_start[b], hi = a.anchor[b];
    bool any = self_tile;
    if (!self_tile)
      for (int j = 0; j < nrows; ++j) any |= (gpos[j] >= lo && gpos[j] < hi);
    if (!any) continue;
    for (int h = g * grp; h < (g + 1) * grp; ++h) {
      __syncthreads();
      for (int idx = tid; idx < kBlock * D; idx += kThreads) {
        const int i = idx / D, c = idx % D;
        const int64_t src = (static_cast<int64_t>(kBlock * b + i) * a.hq + h) * D + c;
        qs[i][c] = Q[src];
        dos[i][c] = dO[src];
      }
      if (tid < kBlock) {
        const int64_t r = static_cast<int64_t>(kBlock * b + tid) * a.hq + h;
        lse_s[tid] = a.lse_in[r];
        del_s[tid] = a.delta[r];
      }
      __syncthreads();
      if (wave == 0) {
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kk = 0; kk < D / 4; ++kk) {
          sc = mma4(ks[l16][4 * kk + q4], qs[l16][4 * kk + q4], sc);
          dp = mma4(vs[l16][4 * kk + q4], dos[l16][4 * kk + q4], dp);
        }
        // lane: keys 4 q4 + r of the tile, query l16
        const float lq = lse_s[l16], dq_ = del_s[l16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 4 * q4 + r;
          const bool allowed = j < nrows && (self_tile || (gpos[j] >= lo && gpos[j] < hi)) && lq != -INFINITY;
          float pv = 0.f, ds = 0.f;
          if (allowed) {
            pv = expf(sc[r] * a.scale - lq);
            ds = pv * (dp[r] - dq_);
          }
          ps[l16][j] = pv;
          dss[l16][j] = ds;
        }
      }
      __syncthreads();
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int dt = wave + 4 * t;
#pragma unroll
        for (int kk = 0; kk < kBlock / 4; ++kk) {
          dv[t] = mma4(dos[4 * kk + q4][16 * dt + l16], ps[4 * kk + q4][l16], dv[t]);
          dk[t] = mma4(qs[4 * kk + q4][16 * dt + l16], dss[4 * kk + q4][l16], dk[t]);
        }
      }
    }
  }
  // lane holds column l16 (a key) of the dcol rows 16 dt + 4 q4 + r
  if (l16 < nrows) {
    float* dK = static_cast<float*>(self_tile ? a.dk_self : a.dk);
    float* dV = static_cast<float*>(self_tile ? a.dv_self : a.dv);
    const int64_t dst = ((row0 + l16) * a.hkv + g) * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * (wave + 4 * t) + 4 * q4 + r;
        dK[dst + c] = a.scale * dk[t][r];
        dV[dst + c] = dv[t][r];
      }
  }
}

template <int D>
hipError_t launch_fwd_f32_d(const AttnArgs& a, hipStream_t s) {
  fwd_f32_kernel<D><<<dim3(a.n_blk, a.hq), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_f32_d(const AttnArgs& a, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (a.flags & SXA_BWD_DELTA) {
    if ((e = launch_delta(a, false, s)) != hipSuccess) return e;
  }
  if (a.flags & SXA_BWD_DQ) {
    dq_f32_kernel<D><<<dim3(a.n_blk, a.hq), kThreads, 0, s>>>(a, (a.flags & SXA_BWD_DQ_OVERWRITE) != 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!(a.flags & SXA_BWD_DKDV)) return hipSuccess;
  const int n_ctx_tiles = static_cast<int>((a.n_loc + kBlock - 1) / kBlock);
  const int n_tiles = n_ctx_tiles + (a.k_self != nullptr ? a.n_blk : 0);
  if (n_tiles == 0) return hipSuccess;
  dkdv_f32_kernel<D><<<dim3(n_tiles, a.hkv), kThreads, 0, s>>>(a, n_ctx_tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_delta(const AttnArgs& a, bool bf16, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * a.hq;
  const dim3 grid(static_cast<unsigned>((rows + kThreads / 16 - 1) / (kThreads / 16)));
  if (bf16) {
    const uint16_t* o = static_cast<const uint16_t*>(a.o_in);
    const uint16_t* d = static_cast<const uint16_t*>(a.dout);
    if (a.d == 64) delta_kernel<uint16_t, 64><<<grid, kThreads, 0, s>>>(o, d, a.lse_in, a.delta, rows);
    else delta_kernel<uint16_t, 128><<<grid, kThreads, 0, s>>>(o, d, a.lse_in, a.delta, rows);
  } else {
    const float* o = static_cast<const float*>(a.o_in);
    const float* d = static_cast<const float*>(a.dout);
    if (a.d == 64) delta_kernel<float, 64><<<grid, kThreads, 0, s>>>(o, d, a.lse_in, a.delta, rows);
    else delta_kernel<float, 128><<<grid, kThreads, 0, s>>>(o, d, a.lse_in, a.delta, rows);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_fwd_f32_d<64>(a, s) : launch_fwd_f32_d<128>(a, s);
}

hipError_t launch_bwd_f32(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_bwd_f32_d<64>(a, s) : launch_bwd_f32_d<128>(a, s);
}

}  // namespace sxa
