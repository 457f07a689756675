// The longest-processing-time-first plan on the device ("Split-KV speeds diffusion
// drafter training...", section "Balance actual attention work": costly chunks first,
// each to the device with the least work among those with room left, every device
// ending with the same chunk count).
//
// The same assignment as the host planner (lpt.cpp), computed by one workgroup from
// the device-resident costs, so that a step needs no round trip through the host:
//   1. rank the chunks by (cost descending, index ascending), in parallel;
//   2. visit them in rank order: each chunk goes to the bin with the least (load,
//      index) among those with fewer than n_chunk / n_bin chunks.  Up to 8 bins with
//      non-negative costs whose total stays below 2^28, eight lanes of one wave hold
//      the bins as 32-bit keys and take the least in three DPP steps; otherwise, up to
//      kScanBins bins, one thread holds them in registers (no memory access or
//      cross-lane step on the chain from one chunk to the next); beyond, one wave's
//      lanes hold the bins and take a wave-wide arg-min;
//   3. write each bin's chunk list in increasing chunk index (the order a stable sort
//      of the chunks by bin gives), with the chunks' global starts and lengths.
#include "internal.h"

namespace sxa {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kScanBins = 32;  // up to this many bins one thread scans them

// The greedy visit for up to NB bins in one thread, the bins' loads and counts in
// registers (bins past n_bin start full, so they are never chosen): a chunk costs one
// unrolled arg-min and one unrolled charge, with no memory access on the chain.
template <int NB>
__device__ __forceinline__ void greedy_scan(int n, int n_bin, int cap, const long long* c_sorted,
                                            const int* ord, int* bin_s, long long* load_s) {
  long long ld[NB];
  int ct[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ld[b] = 0;
    ct[b] = b < n_bin ? 0 : cap;
  }
#pragma unroll 4
  for (int k = 0; k < n; ++k) {
    long long bl = 0x7fffffffffffffffLL;
    int bb = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {  // first least: ties go to the lower index
      const bool better = ct[b] < cap && ld[b] < bl;
      bl = better ? ld[b] : bl;
      bb = better ? b : bb;
    }
    const long long c = c_sorted[k];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      ld[b] += b == bb ? c : 0;
      ct[b] += b == bb ? 1 : 0;
    }
    bin_s[ord[k]] = bb;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (b < n_bin) load_s[b] = ld[b];
}

// Least of the eight values held by each group of eight lanes, left in all eight:
// swap neighbours (DPP quad_perm [1,0,3,2]), then pairs (quad_perm [2,3,0,1]), then
// the two quads (row_half_mirror).
__device__ __forceinline__ uint32_t min8_dpp(uint32_t m) {
  m = min(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0xB1, 0xF, 0xF, false)));
  m = min(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x4E, 0xF, 0xF, false)));
  m = min(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x141, 0xF, 0xF, false)));
  return m;
}

// The greedy visit for up to 8 bins by one full wave.  Lane b < n_bin holds bin b's
// key (load << 3) | b, with bit 31 set once the bin holds cap chunks; every other lane
// holds 0xffffffff.  The least key is the least (load, index) among bins with room
// (a full bin's key exceeds every open one's while the loads stay below 2^28), so a
// chunk costs one three-step DPP minimum, one readfirstlane and the owner's charge.
// Each lane holds one chunk of the current block of 64 (its cost and index), so no
// memory access sits on the chain, and lane k records the bin of the block's chunk k.
// Valid for costs >= 0 whose total is below 2^28; n is a multiple of n_bin, so a bin
// is always open while chunks remain.
__device__ __forceinline__ void greedy_dpp8(int n, int n_bin, int cap, const long long* c_sorted, const int* ord,
                                            int* bin_s, long long* load_s) {
  const int lane = threadIdx.x % 64;
  uint32_t key = lane < n_bin ? static_cast<uint32_t>(lane) : 0xffffffffu;
  int ct = 0;
  for (int k0 = 0; k0 < n; k0 += 64) {
    const int kn = min(64, n - k0);
    const int cl = lane < kn ? static_cast<int>(c_sorted[k0 + lane]) : 0;
    const int ol = lane < kn ? ord[k0 + lane] : 0;
    int mybin = 0;
    for (int k = 0; k < kn; ++k) {
      const uint32_t m = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(min8_dpp(key))));
      const int bb = static_cast<int>(m & 7u);
      const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(cl, k)) << 3;
      if (lane == bb) {
        key += c;
        ct += 1;
        if (ct == cap) key |= 0x80000000u;
      }
      mybin = lane == k ? bb : mybin;
    }
    if (lane < kn) bin_s[ol] = mybin;
  }
  if (lane < n_bin) load_s[lane] = static_cast<long long>((key & 0x7fffffffu) >> 3);
}

__global__ __launch_bounds__(kPlanThreads) void lpt_plan_kernel(const int64_t* __restrict__ cost, int32_t n,
                                                                int32_t n_bin, const int32_t* __restrict__ chunk_gstart,
                                                                const int32_t* __restrict__ chunk_len,
                                                                int32_t* __restrict__ bin_of, int64_t* __restrict__ bin_load,
                                                                int32_t* __restrict__ plan_gstart,
                                                                int32_t* __restrict__ plan_len) {
  __shared__ long long c_s[kMaxPlanChunks];
  __shared__ long long c_sorted[kMaxPlanChunks];  // costs in visiting order
  __shared__ int ord[kMaxPlanChunks];
  __shared__ int bin_s[kMaxPlanChunks];
  __shared__ long long load_s[kMaxPlanBins];
  __shared__ int cnt_s[kMaxPlanBins];
  const int tid = threadIdx.x;
  const int cap = n / n_bin;
  for (int i = tid; i < n; i += kPlanThreads) c_s[i] = cost[i];
  for (int b = tid; b < n_bin; b += kPlanThreads) {
    load_s[b] = 0;
    cnt_s[b] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPlanThreads) {
    const long long ci = c_s[i];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const long long cj = c_s[j];
      rank += (cj > ci) | ((cj == ci) & (j < i));
    }
    ord[rank] = i;
    c_sorted[rank] = ci;
  }
  __shared__ long long tot_s, min_s;
  if (tid < 64) {  // total and least cost: decides whether 32-bit keys hold the loads
    long long t = 0, mn = 0x7fffffffffffffffLL;
    for (int i = tid; i < n; i += 64) {
      const long long c = c_s[i];
      t += c < 0 ? 0 : (c < (1LL << 28) ? c : (1LL << 28));  // clamped: no overflow
      mn = c < mn ? c : mn;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      t += __shfl_xor(t, off, 64);
      const long long o = __shfl_xor(mn, off, 64);
      mn = o < mn ? o : mn;
    }
    if (tid == 0) {
      tot_s = t;
      min_s = mn;
    }
  }
  __syncthreads();
  if (n_bin <= 8 && min_s >= 0 && tot_s < (1LL << 28)) {
    if (tid < 64) greedy_dpp8(n, n_bin, cap, c_sorted, ord, bin_s, load_s);
  } else if (n_bin <= kScanBins) {
    if (tid == 0) {
      if (n_bin <= 8) greedy_scan<8>(n, n_bin, cap, c_sorted, ord, bin_s, load_s);
      else if (n_bin <= 16) greedy_scan<16>(n, n_bin, cap, c_sorted, ord, bin_s, load_s);
      else greedy_scan<kScanBins>(n, n_bin, cap, c_sorted, ord, bin_s, load_s);
    }
  } else if (tid < 64) {
    const int lane = tid;
    for (int k = 0; k < n; ++k) {
      const int c = ord[k];
      long long bl = 0x7fffffffffffffffLL;
      int bb = 0x7fffffff;
      for (int b = lane; b < n_bin; b += 64) {
        const long long lb = load_s[b];
        if (cnt_s[b] < cap && (lb < bl || (lb == bl && b < bb))) {
          bl = lb;
          bb = b;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const long long ol = __shfl_xor(bl, off, 64);
        const int ob = __shfl_xor(bb, off, 64);
        if (ol < bl || (ol == bl && ob < bb)) {
          bl = ol;
          bb = ob;
        }
      }
      // every lane holds the winner; the lane that owns it charges it (LDS accesses
      // of one wave complete in order, so the next chunk sees the update)
      if (bb % 64 == lane) {
        load_s[bb] += c_s[c];
        cnt_s[bb] += 1;
      }
      if (lane == 0) bin_s[c] = bb;
    }
  }
  __syncthreads();
  for (int i = tid; i < n; i += kPlanThreads) {
    const int b = bin_s[i];
    int pos = 0;
#pragma unroll 8
    for (int j = 0; j < i; ++j) pos += bin_s[j] == b;
    bin_of[i] = b;
    plan_gstart[static_cast<int64_t>(b) * cap + pos] = chunk_gstart[i];
    plan_len[static_cast<int64_t>(b) * cap + pos] = chunk_len[i];
  }
  for (int b = tid; b < n_bin; b += kPlanThreads) bin_load[b] = load_s[b];
}

}  // namespace

hipError_t launch_lpt_plan(const int64_t* cost, int32_t n_chunk, int32_t n_bin, const int32_t* chunk_gstart,
                           const int32_t* chunk_len, int32_t* bin_of, int64_t* bin_load, int32_t* plan_gstart,
                           int32_t* plan_len, hipStream_t s) {
  lpt_plan_kernel<<<dim3(1), dim3(kPlanThreads), 0, s>>>(cost, n_chunk, n_bin, chunk_gstart, chunk_len, bin_of,
                                                         bin_load, plan_gstart, plan_len);
  return hipGetLastError();
}

}  // namespace sxa
