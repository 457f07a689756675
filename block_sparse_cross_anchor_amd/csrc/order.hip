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

// Tiles walked by each row group, into cost[0 .. n_groups); glo and ghi are free
// for reuse afterwards.  Ends with a barrier.
__device__ void group_tiles(const AttnArgs& a, int rows_per_group, int n_groups, int* cost, int* glo,
                            int* ghi, int* cgs, int* clen) {
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
}

__global__ __launch_bounds__(kOrderThreads) void row_group_order_kernel(AttnArgs a, int rows_per_group,
                                                                         int n_groups, int32_t* order) {
  __shared__ int cost[kMaxOrderedGroups];
  __shared__ int glo[kMaxOrderedGroups], ghi[kMaxOrderedGroups];
  __shared__ int cgs[kLdsChunks], clen[kLdsChunks];
  group_tiles(a, rows_per_group, n_groups, cost, glo, ghi, cgs, clen);
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

// Exclusive prefix sums of v[0, n) in place, n <= 4 kOrderThreads: per-thread runs,
// a wave-level scan of the run sums, then the wave totals (tmp: kOrderThreads / 64
// ints).  Called by the whole workgroup; ends with a barrier.
__device__ void scan_exclusive(int* v, int n, int* tmp) {
  const int t = threadIdx.x, lane = t % 64, wave = t / 64;
  const int per = (n + kOrderThreads - 1) / kOrderThreads;
  int before[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = t * per + j;
    const int x = (j < per && idx < n) ? v[idx] : 0;
    before[j] = sum;
    sum += x;
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = incl - sum;
  for (int w = 0; w < wave; ++w) base += tmp[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = t * per + j;
    if (j < per && idx < n) v[idx] = base + before[j];
  }
  __syncthreads();
}

constexpr int kLenBuckets = 1024;  // piece lengths are ranked exactly up to this many tiles

// The split forward's plan.  cap = max(kMinSplitTiles, ceil(1.5 total tiles * hkv / n_cu)),
// 1.5 times the mean work of one compute unit (a lower cap also splits groups whose
// pieces then cost more in fixed per-workgroup work than they save; measured and
// modelled on the 64-bin share); a group of T > cap tiles becomes ceil(T / cap)
// pieces, piece k covering tiles [k T / n, (k + 1) T / n) of its walk.  Jobs are
// placed by a counting sort on piece length, longest first (pieces of equal length
// in any order; buckets of cap / kLenBuckets tiles when cap exceeds kLenBuckets), so
// dispatch in index order is longest-first.  Pieces of split groups get consecutive
// slots in group order.  Every pass is parallel over groups or length buckets.
__global__ __launch_bounds__(kOrderThreads) void row_split_plan_kernel(AttnArgs a, int n_groups, RowSplit sp) {
  __shared__ int cost[kMaxOrderedGroups];
  __shared__ int pieces[kMaxOrderedGroups];
  __shared__ int slot[kMaxOrderedGroups], sidx[kMaxOrderedGroups];  // (interval arrays first)
  __shared__ int cgs[kLdsChunks], clen[kLdsChunks];
  __shared__ int hist[kLenBuckets], tmp[kOrderThreads / 64];
  __shared__ unsigned long long total;
  __shared__ int n_split_pieces, n_cut_groups, n_jobs;
  const int tid = threadIdx.x;
  if (tid == 0) {
    total = 0;
    n_split_pieces = 0;
    n_cut_groups = 0;
    n_jobs = 0;
  }
  for (int b = tid; b < kLenBuckets; b += kOrderThreads) hist[b] = 0;
  group_tiles(a, kRowsPerGroup, n_groups, cost, slot, sidx, cgs, clen);
  unsigned long long mine = 0;
  for (int i = tid; i < n_groups; i += kOrderThreads) mine += static_cast<unsigned long long>(cost[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off, 64);
  if (tid % 64 == 0 && mine != 0) atomicAdd(&total, mine);  // one LDS atomic per wave
  __syncthreads();
  const long long want = (3 * static_cast<long long>(total) * a.hkv + 2 * a.n_cu - 1) / (2 * a.n_cu);
  const int cap = static_cast<int>(max<long long>(kMinSplitTiles, min<long long>(want, 0x3fffffff)));
  for (int i = tid; i < n_groups; i += kOrderThreads) {
    const int n = cost[i] > cap ? (cost[i] + cap - 1) / cap : 1;
    pieces[i] = n;
    if (n > 1) {
      atomicAdd(&n_split_pieces, n);
      atomicAdd(&n_cut_groups, 1);
    }
  }
  __syncthreads();
  // both hold by the choice of cap; kept as guards (the grid has max_extra spare slots)
  const bool split_ok = n_split_pieces <= sp.max_pieces && n_split_pieces - n_cut_groups <= sp.max_extra;
  auto bucket = [&](int L) {
    const int b = cap < kLenBuckets ? L : static_cast<int>(static_cast<int64_t>(L) * (kLenBuckets - 1) / cap);
    return kLenBuckets - 1 - min(b, kLenBuckets - 1);  // longest first
  };
  for (int i = tid; i < n_groups; i += kOrderThreads) {
    if (!split_ok) pieces[i] = 1;
    const int n = pieces[i], t = cost[i];
    slot[i] = n > 1 ? n : 0;
    sidx[i] = n > 1 ? 1 : 0;
    for (int k = 0; k < n; ++k)
      atomicAdd(&hist[bucket(static_cast<int>(static_cast<int64_t>(k + 1) * t / n - static_cast<int64_t>(k) * t / n))], 1);
    atomicAdd(&n_jobs, n);
  }
  __syncthreads();
  scan_exclusive(slot, n_groups, tmp);   // first slot of each split group
  scan_exclusive(sidx, n_groups, tmp);   // index among split groups
  scan_exclusive(hist, kLenBuckets, tmp);  // first job of each length bucket
  for (int i = tid; i < n_groups; i += kOrderThreads) {
    const int n = pieces[i], t = cost[i];
    for (int k = 0; k < n; ++k) {
      const int t0 = static_cast<int>(static_cast<int64_t>(k) * t / n);
      const int t1 = static_cast<int>(static_cast<int64_t>(k + 1) * t / n);
      const int job = atomicAdd(&hist[bucket(t1 - t0)], 1);
      sp.jobs[job] = n > 1 ? int4{i, t0, t1, slot[i] + k} : int4{i, 0, 0x7fffffff, -1};
    }
    if (n > 1) sp.groups[sidx[i]] = int4{i, slot[i], n, 0};
  }
  const int n_split_groups = sidx[n_groups - 1] + (pieces[n_groups - 1] > 1 ? 1 : 0);
  for (int x = n_jobs + tid; x < n_groups + sp.max_pieces; x += kOrderThreads) sp.jobs[x] = int4{-1, 0, 0, -1};
  for (int x = n_split_groups + tid; x < sp.max_pieces / 2; x += kOrderThreads) sp.groups[x] = int4{-1, 0, 0, 0};
}

}  // namespace

int64_t row_groups(const AttnArgs& a, int rows_per_group) {
  const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * (a.hq / a.hkv);
  return (rows + rows_per_group - 1) / rows_per_group;
}

int n_compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

int32_t row_split_max_pieces(int32_t hkv, int32_t n_cu) { return max(2, (2 * n_cu + hkv - 1) / hkv); }
int32_t row_split_max_extra(int32_t hkv, int32_t n_cu) { return max(1, (2 * n_cu + 3 * hkv - 1) / (3 * hkv)); }

namespace {
struct SplitLayout {
  int64_t jobs_off, groups_off, lse_off, o_off, bytes;
};
SplitLayout split_layout(int64_t groups, int64_t hkv, int64_t d, int64_t pieces) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  SplitLayout L;
  L.jobs_off = 0;
  L.groups_off = up(16 * (groups + pieces));
  L.lse_off = L.groups_off + up(16 * (pieces / 2));
  L.o_off = L.lse_off + up(4 * pieces * hkv * kRowsPerGroup);
  L.bytes = L.o_off + 4 * pieces * hkv * kRowsPerGroup * d;
  return L;
}
}  // namespace

int64_t row_split_bytes(int32_t n_blk, int32_t hq, int32_t hkv, int32_t d, int32_t n_cu) {
  AttnArgs a;
  a.n_blk = n_blk;
  a.hq = hq;
  a.hkv = hkv;
  const int64_t groups = row_groups(a, kRowsPerGroup);
  if (groups <= 0 || groups > kMaxOrderedGroups) return 0;
  return split_layout(groups, hkv, d, row_split_max_pieces(hkv, n_cu)).bytes;
}

RowSplit row_split_layout(void* ws, const AttnArgs& a) {
  const int32_t pieces = row_split_max_pieces(a.hkv, a.n_cu);
  const SplitLayout L = split_layout(row_groups(a, kRowsPerGroup), a.hkv, a.d, pieces);
  char* b = static_cast<char*>(ws);
  RowSplit sp;
  sp.jobs = reinterpret_cast<int4*>(b + L.jobs_off);
  sp.groups = reinterpret_cast<int4*>(b + L.groups_off);
  sp.part_lse = reinterpret_cast<float*>(b + L.lse_off);
  sp.part_o = reinterpret_cast<float*>(b + L.o_off);
  sp.max_pieces = pieces;
  sp.max_extra = row_split_max_extra(a.hkv, a.n_cu);
  return sp;
}

hipError_t launch_row_split_plan(const AttnArgs& a, const RowSplit& sp, hipStream_t s) {
  const int64_t n = row_groups(a, kRowsPerGroup);
  if (n <= 0 || n > kMaxOrderedGroups) return hipErrorInvalidValue;
  row_split_plan_kernel<<<dim3(1), dim3(kOrderThreads), 0, s>>>(a, static_cast<int>(n), sp);
  return hipGetLastError();
}

hipError_t launch_row_group_order(const AttnArgs& a, int rows_per_group, int32_t* order, hipStream_t s) {
  const int64_t n = row_groups(a, rows_per_group);
  if (n <= 0 || n > kMaxOrderedGroups) return hipSuccess;
  row_group_order_kernel<<<dim3(1), dim3(kOrderThreads), 0, s>>>(a, rows_per_group, static_cast<int>(n), order);
  return hipGetLastError();
}

}  // namespace sxa
