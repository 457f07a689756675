// Realised attention cost per contiguous context chunk.
//
// Split-KV prices each context chunk by the attention work that lands on it; every
// device holds all query blocks' metadata, so each can count it for every chunk
// ("Split-KV speeds diffusion drafter training...", section "Balance actual
// attention work").  Block b's B query
// tokens may read keys [sample_start[b], anchor[b]); the cost of chunk c is the
// number of such (query token, key) pairs with the key inside the chunk, i.e.
// B * sum_b |[sample_start[b], anchor[b]) intersect chunk c|, computed exactly in
// int64.  One workgroup per chunk; each thread intersects a strided subset of the
// blocks' intervals with the chunk, then a workgroup reduction sums them.
#include "device_common.h"
#include "internal.h"

namespace sxa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void chunk_cost_kernel(
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ sample_start, int32_t n_blk,
    int32_t n_ctx, int32_t chunk_size, int64_t* __restrict__ cost) {
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * chunk_size;
  const int64_t c1 = min(c0 + chunk_size, static_cast<int64_t>(n_ctx));
  int64_t acc = 0;
  for (int b = threadIdx.x; b < n_blk; b += kThreads) {
    const int64_t lo = max(static_cast<int64_t>(sample_start[b]), c0);
    const int64_t hi = min(static_cast<int64_t>(anchor[b]), c1);
    acc += hi > lo ? hi - lo : 0;
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  __shared__ int64_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot += part[w];
    cost[blockIdx.x] = tot * kBlock;
  }
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(void* p, int64_t n_words, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  const int64_t want = (n_words + kThreads - 1) / kThreads;
  const int64_t blocks = want < 4096 ? want : 4096;
  zero_words_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(
      static_cast<uint32_t*>(p), n_words);
  return hipGetLastError();
}

hipError_t launch_chunk_cost(const int32_t* anchor, const int32_t* sample_start, int32_t n_blk,
                             int32_t n_ctx, int32_t chunk_size, int64_t* cost, hipStream_t s) {
  const int64_t n_chunk = (static_cast<int64_t>(n_ctx) + chunk_size - 1) / chunk_size;
  if (n_chunk == 0) return hipSuccess;
  chunk_cost_kernel<<<dim3(static_cast<unsigned>(n_chunk)), dim3(kThreads), 0, s>>>(
      anchor, sample_start, n_blk, n_ctx, chunk_size, cost);
  return hipGetLastError();
}

}  // namespace sxa
