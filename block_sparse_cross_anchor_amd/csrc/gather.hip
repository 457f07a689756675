// Context redistribution: copy the rows of the listed chunks of a packed context
// tensor back to back into a local buffer.  After the planner has assigned chunks
// to devices, each device's share of the context is moved to it once per step
// ("Split-KV speeds diffusion drafter training...", section "Balance actual
// attention work").  A pure HBM-bound copy: workgroup (c, s) streams stripe s of
// chunk c with 16-byte loads and stores.
#include "device_common.h"
#include "internal.h"

namespace sxa {
namespace {

constexpr int kThreads = 256;

constexpr int kPerThread = 4;  // 16-byte copies per thread, all loads issued before the stores

// Workgroup (c, s) copies the s-th run of kThreads * kPerThread 16-byte units of chunk c.
__global__ __launch_bounds__(kThreads) void gather_kernel(const uint8_t* __restrict__ src,
                                                          int64_t row_bytes,
                                                          const int32_t* __restrict__ cgs,
                                                          const int32_t* __restrict__ clen,
                                                          int64_t n_dst_rows,
                                                          uint8_t* __restrict__ dst) {
  const int c = blockIdx.x;
  int64_t off = 0;
  for (int i = 0; i < c; ++i) off += clen[i];
  const int64_t rows = min(static_cast<int64_t>(clen[c]), n_dst_rows - off);
  if (rows <= 0) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(cgs[c]) * row_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(dst + off * row_bytes);
  const int64_t n16 = rows * row_bytes / 16;
  const int64_t i0 = static_cast<int64_t>(blockIdx.y) * kThreads * kPerThread + threadIdx.x;
  for (int64_t base = i0; base < n16; base += static_cast<int64_t>(gridDim.y) * kThreads * kPerThread) {
    u32x4 v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (base + j * kThreads < n16) v[j] = s[base + j * kThreads];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      if (base + j * kThreads < n16) d[base + j * kThreads] = v[j];
  }
}

}  // namespace

hipError_t launch_context_gather(const void* src, int64_t row_bytes, const int32_t* chunk_gstart,
                                 const int32_t* chunk_len, int32_t n_chunk, int64_t n_dst_rows,
                                 void* dst, hipStream_t s) {
  // runs per chunk: enough for the mean chunk length (longer chunks loop)
  const int64_t per_chunk16 = (n_dst_rows + n_chunk - 1) / n_chunk * row_bytes / 16;
  int64_t stripes = (per_chunk16 + kThreads * kPerThread - 1) / (kThreads * kPerThread);
  stripes = stripes < 1 ? 1 : (stripes > 65535 ? 65535 : stripes);
  gather_kernel<<<dim3(static_cast<unsigned>(n_chunk), static_cast<unsigned>(stripes)), dim3(kThreads), 0,
                  s>>>(static_cast<const uint8_t*>(src), row_bytes, chunk_gstart, chunk_len, n_dst_rows,
                       static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

}  // namespace sxa
