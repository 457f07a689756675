// Exact log-sum-exp merge of attention partials.
//
// Split-KV merges the per-shard partial outputs from their normalisation
// statistics so that the original attention is reconstructed exactly
// ("Split-KV speeds diffusion drafter training...", section "Exchange the smaller
// side").  For one row with partial statistics lse_p and outputs O_p:
//   m = max_p lse_p,  lse = m + ln sum_p exp(lse_p - m),  O = sum_p exp(lse_p - lse) O_p.
// Partials with lse_p = -inf are skipped without reading their O_p.
//
// The kernel is HBM-bound: it streams every live O_p row once, with non-temporal
// loads (each row is read exactly once; 64-way: 5.3 -> 5.7 TB/s measured).  16 lanes own one row
// (each lane D/16 consecutive elements, 16 B for bf16 at D = 128), so each partial
// row is one fully coalesced 256 B (bf16) segment.  The statistics pass reads the
// P lse values of the row (strided by `rows`); the streaming pass issues the loads
// of 8 partials before their sums.  With more than 8 partials it walks only the
// live ones (a bit mask per row), so empty partials take no slot of a batch.
#include "device_common.h"
#include "internal.h"

namespace sxa {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;
constexpr int kMaxBatch = 8;

template <typename T, int EPL>
struct Vec;
template <>
struct Vec<uint16_t, 8> {
  u32x4 raw;
  __device__ __forceinline__ void load(const uint16_t* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = raw[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Vec<uint16_t, 4> {
  u32x2 raw;
  __device__ __forceinline__ void load(const uint16_t* p) { raw = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = raw[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Vec<uint16_t, 16> {
  u32x4 raw[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    raw[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    raw[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
  }
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = raw[i >> 3][(i >> 1) & 3];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <int EPL>
struct Vec<float, EPL> {
  f32x4 raw[EPL / 4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) raw[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + i);
  }
  __device__ __forceinline__ float get(int i) const { return raw[i >> 2][i & 3]; }
};

template <typename TOut, int EPL>
__device__ __forceinline__ void store_row(TOut* p, const float* x);
template <>
__device__ __forceinline__ void store_row<float, 4>(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
template <>
__device__ __forceinline__ void store_row<float, 8>(float* p, const float* x) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{x[0], x[1], x[2], x[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{x[4], x[5], x[6], x[7]};
}
template <>
__device__ __forceinline__ void store_row<float, 16>(float* p, const float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    reinterpret_cast<f32x4*>(p)[i] = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
}
template <int EPL>
__device__ __forceinline__ void store_bf16_row(uint16_t* p, const float* x) {
  uint32_t w[EPL / 2];
#pragma unroll
  for (int i = 0; i < EPL / 2; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i + 1])) << 16);
  if constexpr (EPL == 4) {
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
  } else {
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i)
      reinterpret_cast<u32x4*>(p)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  }
}
template <>
__device__ __forceinline__ void store_row<uint16_t, 4>(uint16_t* p, const float* x) { store_bf16_row<4>(p, x); }
template <>
__device__ __forceinline__ void store_row<uint16_t, 8>(uint16_t* p, const float* x) { store_bf16_row<8>(p, x); }
template <>
__device__ __forceinline__ void store_row<uint16_t, 16>(uint16_t* p, const float* x) { store_bf16_row<16>(p, x); }

template <typename TIn, typename TOut, int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(const TIn* __restrict__ o_parts,
                                                           const float* __restrict__ lse_parts,
                                                           int32_t n_parts, int64_t rows,
                                                           TOut* __restrict__ o_out,
                                                           float* __restrict__ lse_out) {
  constexpr int EPL = D / kLanesPerRow;
  constexpr int kBatch = kMaxBatch;  // loads issued before their sums
  const int lane = threadIdx.x % kLanesPerRow;
  const int grp_shift = (threadIdx.x % 64) & ~(kLanesPerRow - 1);  // this row's lanes in the wave
  const int64_t row_raw = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const bool live_row = row_raw < rows;
  const int64_t row = live_row ? row_raw : rows - 1;  // keep every lane in the shuffles

  // statistics: max, then sum of exp(lse_p - m), 16 lanes stride over the partials
  float m = -INFINITY;
  for (int p = lane; p < n_parts; p += kLanesPerRow) m = fmaxf(m, lse_parts[p * rows + row]);
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kLanesPerRow));
  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.f;
    for (int p = lane; p < n_parts; p += kLanesPerRow) s += __expf(lse_parts[p * rows + row] - m);
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, kLanesPerRow);
    lse = m + __logf(s);
  }
  const TIn* base = o_parts + row * D + lane * EPL;
  const int64_t pstride = rows * D;
  if (n_parts <= kBatch) {
    // one batch: every partial's load issued before the sums (empty ones skipped)
    if (lse != -INFINITY) {
      Vec<TIn, EPL> x[kBatch];
      float w[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float l = j < n_parts ? lse_parts[j * rows + row] : -INFINITY;
        w[j] = l == -INFINITY ? 0.f : __expf(l - lse);
        if (w[j] != 0.f) x[j].load(base + j * pstride);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (w[j] != 0.f) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) acc[i] = fmaf(w[j], x[j].get(i), acc[i]);
        }
      }
    }
  } else {
    // 64 partials at a time: the row's live partials (finite lse) as a bit mask,
    // then their O rows in ascending order, kBatch loads issued before their sums.
    // Empty partials are never read and take no slot of a batch.  The 16 lanes of a
    // row hold the same mask, so the loops below are uniform within the row.
    for (int c0 = 0; c0 < n_parts; c0 += 64) {
      uint64_t mask = 0;
#pragma unroll
      for (int k = 0; k < 64 / kLanesPerRow; ++k) {
        const int p = c0 + kLanesPerRow * k + lane;
        const bool live = lse != -INFINITY && p < n_parts && lse_parts[p * rows + row] != -INFINITY;
        mask |= ((__ballot(live) >> grp_shift) & ((uint64_t{1} << kLanesPerRow) - 1)) << (kLanesPerRow * k);
      }
      while (mask != 0) {
        Vec<TIn, EPL> x[kBatch];
        float w[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          w[j] = 0.f;
          if (mask != 0) {
            const int p = c0 + __builtin_ctzll(mask);
            mask &= mask - 1;
            w[j] = __expf(lse_parts[p * rows + row] - lse);
            x[j].load(base + p * pstride);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (w[j] != 0.f) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] = fmaf(w[j], x[j].get(i), acc[i]);
          }
        }
      }
    }
  }
  if (live_row) {
    store_row<TOut, EPL>(o_out + row * D + lane * EPL, acc);
    if (lane == 0) lse_out[row] = lse;
  }
}

template <typename TIn, typename TOut>
hipError_t launch_typed(const void* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows,
                        int32_t d, void* o_out, float* lse_out, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const TIn* in = static_cast<const TIn*>(o_parts);
  TOut* out = static_cast<TOut*>(o_out);
  switch (d) {
    case 64:
      combine_kernel<TIn, TOut, 64><<<grid, kThreads, 0, s>>>(in, lse_parts, n_parts, rows, out, lse_out);
      break;
    case 128:
      combine_kernel<TIn, TOut, 128><<<grid, kThreads, 0, s>>>(in, lse_parts, n_parts, rows, out, lse_out);
      break;
    case 256:
      combine_kernel<TIn, TOut, 256><<<grid, kThreads, 0, s>>>(in, lse_parts, n_parts, rows, out, lse_out);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* o_parts, bool part_bf16, const float* lse_parts,
                          int32_t n_parts, int64_t rows, int32_t d, void* o_out, bool out_bf16,
                          float* lse_out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (part_bf16) {
    return out_bf16 ? launch_typed<uint16_t, uint16_t>(o_parts, lse_parts, n_parts, rows, d, o_out, lse_out, s)
                    : launch_typed<uint16_t, float>(o_parts, lse_parts, n_parts, rows, d, o_out, lse_out, s);
  }
  return out_bf16 ? launch_typed<float, uint16_t>(o_parts, lse_parts, n_parts, rows, d, o_out, lse_out, s)
                  : launch_typed<float, float>(o_parts, lse_parts, n_parts, rows, d, o_out, lse_out, s);
}

}  // namespace sxa
