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
// index ascending).
#include "internal.h"

namespace sxa {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kTileKeys = 64;

__global__ __launch_bounds__(kOrderThreads) void row_group_order_kernel(AttnArgs a, int rows_per_group,
                                                                         int n_groups, int32_t* order) {
  __shared__ int cost[kMaxOrderedGroups];
  const int grp = a.hq / a.hkv;
  const int64_t R = static_cast<int64_t>(a.n_blk) * kBlock * grp;
  for (int i = threadIdx.x; i < n_groups; i += kOrderThreads) {
    const int64_t r0 = static_cast<int64_t>(i) * rows_per_group;
    const int64_t r1 = min(r0 + rows_per_group, R) - 1;
    const int b0 = static_cast<int>(r0 / grp / kBlock), b1 = static_cast<int>(r1 / grp / kBlock);
    int lo = 0x7fffffff, hi = -0x7fffffff;
    for (int b = b0; b <= b1; ++b) {
      lo = min(lo, a.sample_start[b]);
      hi = max(hi, a.anchor[b]);
    }
    int n = a.k_self ? (kBlock * (b1 - b0 + 1) + kTileKeys - 1) / kTileKeys : 0;
    for (int c = 0; c < a.n_chunk; ++c) {
      const int gs = a.chunk_gstart[c], len = a.chunk_len[c];
      const int s = max(lo, gs), e = min(hi, gs + len);
      if (s < e) n += (e - gs + kTileKeys - 1) / kTileKeys - (s - gs) / kTileKeys;
    }
    cost[i] = n;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_groups; i += kOrderThreads) {
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
