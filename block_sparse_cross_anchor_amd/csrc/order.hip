// Dispatch order of query row groups, most work first.
//
// The forward and dQ kernels give each workgroup 256 consecutive query rows of one
// kv head and walk the 64-key tiles that the rows' blocks may read: the own-block
// tiles and, in every local chunk, the tiles that meet [min sample start, max
// anchor) of the group's blocks.  That count differs by several times between row
// groups (a block late in a long sample reads far more context), and the hardware
// hands workgroups to compute units in index order, so dispatching the heavy groups
// first approximates longest-processing-time-first scheduling and shortens the tail.
// One workgroup computes every group's tile count and ranks them (count descending,
// index ascending).  Its passes are parallel over blocks, then over (group, chunk)
// pairs, so the metadata is read in one round of independent loads.
#include "internal.h"

namespace sxa {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kTileKeys = 64;
constexpr int kLdsChunks = 1024;  // chunk metadata staged in LDS up to this many chunks

__global__ __launch_bounds__(kOrderThreads) void row_group_order_kernel(AttnArgs a, int rows_per_group,
                                                                         int n_groups, int32_t* order) {
  __shared__ int cost[kMaxOrderedGroups];
  __shared__ int glo[kMaxOrderedGroups], ghi[kMaxOrderedGroups];
  __shared__ int cgs[kLdsChunks], clen[kLdsChunks];
  const int tid = threadIdx.x;
  const int grp = a.hq / a.hkv;
  const int64_t R = static_cast<int64_t>(a.n_blk) * kBlock * grp;
  const bool lds_chunks = a.n_chunk <= kLdsChunks;
  for (int i = tid; i < n_groups; i += kOrderThreads) {
    glo[i] = 0x7fffffff;
    ghi[i] = -0x7fffffff;
    // own-block tiles of the group's blocks
    const int64_t r0 = static_cast<int64_t>(i) * rows_per_group;
    const int64_t r1 = min(r0 + rows_per_group, R) - 1;
    const int b0 = static_cast<int>(r0 / grp / kBlock), b1 = static_cast<int>(r1 / grp / kBlock);
    cost[i] = a.k_self ? (kBlock * (b1 - b0 + 1) + kTileKeys - 1) / kTileKeys : 0;
  }
  if (lds_chunks)
    for (int c = tid; c < a.n_chunk; c += kOrderThreads) {
      cgs[c] = a.chunk_gstart[c];
      clen[c] = a.chunk_len[c];
    }
  __syncthreads();
  // key interval [min sample start, max anchor) of each group's blocks
  for (int b = tid; b < a.n_blk; b += kOrderThreads) {
    const int lo = a.sample_start[b], hi = a.anchor[b];
    const int64_t r0 = static_cast<int64_t>(b) * kBlock * grp, r1 = r0 + kBlock * grp - 1;
    for (int64_t i = r0 / rows_per_group; i <= r1 / rows_per_group; ++i) {
      atomicMin(&glo[i], lo);
      atomicMax(&ghi[i], hi);
    }
  }
  __syncthreads();
  // context tiles: (group, chunk) pairs
  const int64_t pairs = static_cast<int64_t>(n_groups) * a.n_chunk;
  for (int64_t x = tid; x < pairs; x += kOrderThreads) {
    const int i = static_cast<int>(x / a.n_chunk), c = static_cast<int>(x % a.n_chunk);
    const int gs = lds_chunks ? cgs[c] : a.chunk_gstart[c];
    const int len = lds_chunks ? clen[c] : a.chunk_len[c];
    const int s = max(glo[i], gs), e = min(ghi[i], gs + len);
    if (s < e) atomicAdd(&cost[i], (e - gs + kTileKeys - 1) / kTileKeys - (s - gs) / kTileKeys);
  }
  __syncthreads();
  for (int i = tid; i < n_groups; i += kOrderThreads) {
    const int c = cost[i];
    int rank = 0;
    for (int j = 0; j < n_groups; ++j) {
      const int cj = cost[j];
      rank += (cj > c) | ((cj == c) & (j < i));
    }
    order[rank] = i;
  }
}

}  // namespace

int64_t row_groups(const AttnArgs& a, int rows_per_group) {
  const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * (a.hq / a.hkv);
  return (rows + rows_per_group - 1) / rows_per_group;
}

hipError_t launch_row_group_order(const AttnArgs& a, int rows_per_group, int32_t* order, hipStream_t s) {
  const int64_t n = row_groups(a, rows_per_group);
  if (n <= 0 || n > kMaxOrderedGroups) return hipSuccess;
  row_group_order_kernel<<<dim3(1), dim3(kOrderThreads), 0, s>>>(a, rows_per_group, static_cast<int>(n), order);
  return hipGetLastError();
}

}  // namespace sxa
