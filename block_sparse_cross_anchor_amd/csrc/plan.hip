// The longest-processing-time-first plan on the device ("Split-KV speeds diffusion
// drafter training...", section "Balance actual attention work": costly chunks first,
// each to the device with the least work among those with room left, every device
// ending with the same chunk count).
//
// The same assignment as the host planner (lpt.cpp), computed by one workgroup from
// the device-resident costs, so that a step needs no round trip through the host:
//   1. rank the chunks by (cost descending, index ascending), in parallel;
//   2. visit them in rank order: each chunk goes to the bin with the least (load,
//      index) among those with fewer than n_chunk / n_bin chunks.  Up to kScanBins
//      bins one thread holds them in registers (no memory access or cross-lane step on
//      the chain from one chunk to the next); beyond, one wave's lanes hold the bins
//      and take a wave-wide arg-min;
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
  __syncthreads();
  if (n_bin <= kScanBins) {
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
