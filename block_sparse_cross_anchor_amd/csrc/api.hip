// C-ABI entry points of libsxattn (declared in include/sxattn.h): host-side
// argument validation, kernel selection and launch on the caller's stream.
// Every status other than SXA_OK leaves a message in a thread-local buffer that
// sxa_last_error() returns.  No C++ exception crosses the ABI.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace sxa {
int lpt_assign_host(const int64_t* cost, int32_t n_chunk, int32_t n_bin, int32_t* bin_of_chunk,
                    int64_t* bin_load);
}

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SXA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SXA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(sxa_dtype t) { return t == SXA_F32 || t == SXA_BF16; }

// Shared validation of the attention arguments; fills `a` on success.
int check_attn(const void* q, const void* k, const void* v, sxa_dtype in_dtype, int32_t n_blk,
               int32_t block_size, int32_t hq, int32_t hkv, int32_t d, float scale,
               const int32_t* anchor, const int32_t* sample_start, const int32_t* chunk_gstart,
               const int32_t* chunk_len, int32_t n_chunk, int64_t n_loc, const void* k_self,
               const void* v_self, sxa::AttnArgs& a) {
  if (!dtype_ok(in_dtype)) return fail(SXA_EINVAL, "in_dtype %d is not a valid sxa_dtype", in_dtype);
  if (block_size != sxa::kBlock)
    return fail(SXA_EUNSUPPORTED, "block_size %d is not supported (only 16)", block_size);
  if (d != 64 && d != 128) return fail(SXA_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d);
  if (n_blk < 0) return fail(SXA_EINVAL, "n_blk must be >= 0 (got %d)", n_blk);
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0)
    return fail(SXA_EINVAL, "hq (%d) must be a positive multiple of hkv (%d)", hq, hkv);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(SXA_EINVAL, "scale must be positive and finite (got %g)", static_cast<double>(scale));
  if (n_chunk < 0) return fail(SXA_EINVAL, "n_chunk must be >= 0 (got %d)", n_chunk);
  if (n_loc < 0) return fail(SXA_EINVAL, "n_loc must be >= 0");
  if (n_chunk == 0 && n_loc != 0) return fail(SXA_EINVAL, "n_loc must be 0 when n_chunk is 0");
  if (static_cast<int64_t>(n_blk) * sxa::kBlock * hq * d >= (int64_t{1} << 40))
    return fail(SXA_EINVAL, "query tensor too large");
  if (static_cast<int64_t>(n_blk) * sxa::kBlock * hq >= (int64_t{1} << 29))
    return fail(SXA_EUNSUPPORTED, "n_blk * 16 * hq must be below 2^29 query rows");
  if (hkv > 4096)  // per-lane byte offsets of a key tile's rows are 24-bit products
    return fail(SXA_EUNSUPPORTED, "hkv %d is above the supported 4096", hkv);
  if ((k_self == nullptr) != (v_self == nullptr))
    return fail(SXA_EINVAL, "k_self and v_self must be both NULL or both non-NULL");
  if (n_blk > 0 && (q == nullptr || anchor == nullptr || sample_start == nullptr))
    return fail(SXA_EINVAL, "q, anchor and sample_start must not be NULL");
  if (n_chunk > 0 && (chunk_gstart == nullptr || chunk_len == nullptr))
    return fail(SXA_EINVAL, "chunk_gstart and chunk_len must not be NULL when n_chunk > 0");
  if (n_loc > 0 && (k == nullptr || v == nullptr)) return fail(SXA_EINVAL, "k and v must not be NULL");
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_self = k_self;
  a.v_self = v_self;
  a.n_blk = n_blk;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.scale = scale;
  a.anchor = anchor;
  a.sample_start = sample_start;
  a.chunk_gstart = chunk_gstart;
  a.chunk_len = chunk_len;
  a.n_chunk = n_chunk;
  a.n_loc = n_loc;
  return SXA_OK;
}

// Scratch of sparse_xattn_fwd_noalloc: the forward's ranked dispatch order (one int32
// per query row group of 256 rows, up to kMaxOrderedGroups) in a file-scope device
// array, so that the call allocates nothing.  Every device that runs the library holds
// its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is looked up once per device
// with hipGetSymbolAddress and only that address is passed to kernels.
constexpr int kNoallocScratchInts = sxa::kMaxOrderedGroups;
static __device__ __align__(256) int32_t scratch[kNoallocScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of `scratch` on the current device (looked up on its first use there).
int scratch_on_current_device(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SXA_EUNSUPPORTED, "device index %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(SXA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return SXA_OK;
}

}  // namespace

extern "C" {

const char* sxa_last_error(void) { return g_err; }

int sparse_xattn_fwd(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                     int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                     float scale, const int32_t* anchor, const int32_t* sample_start,
                     const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                     int64_t n_loc, const void* k_self, const void* v_self, void* o,
                     sxa_dtype o_dtype, float* lse, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  sxa::AttnArgs a;
  int st = check_attn(q, k, v, in_dtype, n_blk, block_size, hq, hkv, d, scale, anchor,
                      sample_start, chunk_gstart, chunk_len, n_chunk, n_loc, k_self, v_self, a);
  if (st != SXA_OK) return st;
  if (!dtype_ok(o_dtype)) return fail(SXA_EINVAL, "o_dtype %d is not a valid sxa_dtype", o_dtype);
  if (in_dtype == SXA_F32 && o_dtype != SXA_F32)
    return fail(SXA_EUNSUPPORTED, "float32 inputs need a float32 output");
  if (n_blk > 0 && (o == nullptr || lse == nullptr)) return fail(SXA_EINVAL, "o and lse must not be NULL");
  a.o = o;
  a.o_bf16 = o_dtype == SXA_BF16;
  a.lse = lse;
  if (workspace_bytes < 0) return fail(SXA_EINVAL, "workspace_bytes must be >= 0");
  const int64_t need = sparse_xattn_fwd_workspace_bytes(n_blk, hq, hkv);
  if (workspace != nullptr && need > 0 && workspace_bytes >= need) a.rg_order = static_cast<int32_t*>(workspace);
  a.row_split = nullptr;
  a.n_cu = 0;
  if (workspace != nullptr && in_dtype == SXA_BF16) {
    const int32_t n_cu = sxa::n_compute_units();
    const int64_t split = sxa::row_split_bytes(n_blk, hq, hkv, d, n_cu);
    if (split > 0 && workspace_bytes >= split) {
      a.row_split = workspace;
      a.n_cu = n_cu;
    }
  }
  if (n_blk == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(in_dtype == SXA_BF16 ? sxa::launch_fwd_bf16(a, s) : sxa::launch_fwd_f32(a, s),
                    "sparse_xattn_fwd launch");
}

int sparse_xattn_fwd_noalloc(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                             int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                             float scale, const int32_t* anchor, const int32_t* sample_start,
                             const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                             int64_t n_loc, const void* k_self, const void* v_self, void* o,
                             sxa_dtype o_dtype, float* lse, void* stream) {
  sxa::AttnArgs a;
  int st = check_attn(q, k, v, in_dtype, n_blk, block_size, hq, hkv, d, scale, anchor,
                      sample_start, chunk_gstart, chunk_len, n_chunk, n_loc, k_self, v_self, a);
  if (st != SXA_OK) return st;
  if (!dtype_ok(o_dtype)) return fail(SXA_EINVAL, "o_dtype %d is not a valid sxa_dtype", o_dtype);
  if (in_dtype == SXA_F32 && o_dtype != SXA_F32)
    return fail(SXA_EUNSUPPORTED, "float32 inputs need a float32 output");
  if (n_blk > 0 && (o == nullptr || lse == nullptr)) return fail(SXA_EINVAL, "o and lse must not be NULL");
  const int64_t groups = sxa::row_groups(a, sxa::kRowsPerGroup);
  if (groups > kNoallocScratchInts)
    return fail(SXA_EUNSUPPORTED,
                "sparse_xattn_fwd_noalloc: %lld query row groups of 256 rows per kv head exceed the "
                "static scratch of %d (use sparse_xattn_fwd with a workspace)",
                static_cast<long long>(groups), kNoallocScratchInts);
  a.o = o;
  a.o_bf16 = o_dtype == SXA_BF16;
  a.lse = lse;
  a.row_split = nullptr;
  a.n_cu = 0;
  if (n_blk == 0) return ok();
  if (in_dtype == SXA_BF16) {
    int32_t* order = nullptr;
    if ((st = scratch_on_current_device(&order)) != SXA_OK) return st;
    a.rg_order = order;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(in_dtype == SXA_BF16 ? sxa::launch_fwd_bf16(a, s) : sxa::launch_fwd_f32(a, s),
                    "sparse_xattn_fwd_noalloc launch");
}

int sparse_xattn_bwd(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                     int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                     float scale, const int32_t* anchor, const int32_t* sample_start,
                     const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                     int64_t n_loc, const void* k_self, const void* v_self, const void* o,
                     const void* dout, const float* lse, float* delta_ws, float* dq_accum,
                     void* dk, void* dv, void* dk_self, void* dv_self, void* workspace,
                     int64_t workspace_bytes, int32_t flags, void* stream) {
  sxa::AttnArgs a;
  int st = check_attn(q, k, v, in_dtype, n_blk, block_size, hq, hkv, d, scale, anchor,
                      sample_start, chunk_gstart, chunk_len, n_chunk, n_loc, k_self, v_self, a);
  if (st != SXA_OK) return st;
  constexpr int32_t kAll = SXA_BWD_DELTA | SXA_BWD_DQ | SXA_BWD_DKDV;
  if ((flags & kAll) == 0) flags |= kAll;  // no phase named: every phase
  if (flags & ~(kAll | SXA_BWD_DQ_OVERWRITE | SXA_BWD_DKDV_BF16)) return fail(SXA_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & SXA_BWD_DKDV_BF16) && in_dtype != SXA_BF16)
    return fail(SXA_EUNSUPPORTED, "bf16 key/value gradients need bf16 inputs");
  if (n_blk > 0 && (o == nullptr || dout == nullptr || lse == nullptr || delta_ws == nullptr))
    return fail(SXA_EINVAL, "o, dout, lse and delta_ws must not be NULL");
  if (n_blk > 0 && (flags & SXA_BWD_DQ) && dq_accum == nullptr)
    return fail(SXA_EINVAL, "dq_accum must not be NULL");
  if ((flags & SXA_BWD_DKDV) && n_loc > 0 && (dk == nullptr || dv == nullptr))
    return fail(SXA_EINVAL, "dk and dv must not be NULL");
  if ((flags & SXA_BWD_DKDV) && k_self != nullptr && (dk_self == nullptr || dv_self == nullptr))
    return fail(SXA_EINVAL, "dk_self and dv_self must not be NULL when k_self is given");
  a.o_in = o;
  a.dout = dout;
  a.lse_in = lse;
  a.delta = delta_ws;
  a.dq = dq_accum;
  a.dk = dk;
  a.dv = dv;
  a.dk_self = dk_self;
  a.dv_self = dv_self;
  a.flags = flags;
  if (workspace_bytes < 0) return fail(SXA_EINVAL, "workspace_bytes must be >= 0");
  const int64_t need = sxa::bwd_workspace_bytes(n_blk, n_loc, hq, hkv, d);
  a.workspace = (workspace != nullptr && need > 0 && workspace_bytes >= need) ? workspace : nullptr;
  a.workspace_bytes = workspace_bytes;
  if (a.workspace != nullptr && in_dtype == SXA_BF16 && (flags & SXA_BWD_DQ)) {
    const int32_t n_cu = sxa::n_compute_units();
    const int64_t split = sxa::row_split_bytes(n_blk, hq, hkv, d, n_cu);
    const int64_t base = (need + 255) / 256 * 256;
    if (split > 0 && workspace_bytes >= base + split) {  // the split dQ schedule's plan and slots
      a.row_split = static_cast<char*>(workspace) + base;
      a.n_cu = n_cu;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_blk == 0) {
    if (!(flags & SXA_BWD_DKDV)) return ok();
    // no query: the gradients of the local keys/values are zero
    const int64_t kv_words = n_loc * hkv * d / ((flags & SXA_BWD_DKDV_BF16) ? 2 : 1);  // 32-bit words
    hipError_t e = sxa::launch_zero_words(dk, kv_words, s);
    if (e == hipSuccess) e = sxa::launch_zero_words(dv, kv_words, s);
    return hip_status(e, "sparse_xattn_bwd zero fill");
  }
  return hip_status(in_dtype == SXA_BF16 ? sxa::launch_bwd_bf16(a, s) : sxa::launch_bwd_f32(a, s),
                    "sparse_xattn_bwd launch");
}

int64_t sparse_xattn_fwd_workspace_bytes(int32_t n_blk, int32_t hq, int32_t hkv) {
  if (n_blk < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return 0;
  sxa::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.n_blk = n_blk;
  a.hq = hq;
  a.hkv = hkv;
  const int64_t groups = sxa::row_groups(a, sxa::kRowsPerGroup);
  return 4 * (groups < sxa::kMaxOrderedGroups ? groups : sxa::kMaxOrderedGroups);
}

int64_t sparse_xattn_fwd_split_workspace_bytes(int32_t n_blk, int32_t hq, int32_t hkv, int32_t d) {
  if (n_blk < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || (d != 64 && d != 128)) return 0;
  return sxa::row_split_bytes(n_blk, hq, hkv, d, sxa::n_compute_units());
}

int64_t sparse_xattn_bwd_split_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv, int32_t d) {
  if (n_blk < 0 || n_loc < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || (d != 64 && d != 128)) return 0;
  const int64_t need = sxa::bwd_workspace_bytes(n_blk, n_loc, hq, hkv, d);
  const int64_t split = sxa::row_split_bytes(n_blk, hq, hkv, d, sxa::n_compute_units());
  if (need <= 0 || split <= 0) return 0;
  return (need + 255) / 256 * 256 + split;
}

int64_t sparse_xattn_bwd_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv, int32_t d) {
  if (n_blk < 0 || n_loc < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || (d != 64 && d != 128)) return 0;
  return sxa::bwd_workspace_bytes(n_blk, n_loc, hq, hkv, d);
}

int lse_combine(const void* o_parts, sxa_dtype part_dtype, const float* lse_parts,
                int32_t n_parts, int64_t rows, int32_t d, void* o_out, sxa_dtype out_dtype,
                float* lse_out, void* stream) {
  if (!dtype_ok(part_dtype) || !dtype_ok(out_dtype)) return fail(SXA_EINVAL, "invalid dtype");
  if (n_parts < 0 || rows < 0) return fail(SXA_EINVAL, "n_parts and rows must be >= 0");
  if (d != 64 && d != 128 && d != 256) return fail(SXA_EUNSUPPORTED, "d %d is not supported (64, 128, 256)", d);
  if (rows > 0 && (o_out == nullptr || lse_out == nullptr)) return fail(SXA_EINVAL, "outputs must not be NULL");
  if (rows > 0 && n_parts > 0 && (o_parts == nullptr || lse_parts == nullptr))
    return fail(SXA_EINVAL, "inputs must not be NULL");
  if (rows >= (int64_t{1} << 34)) return fail(SXA_EINVAL, "rows too large");
  if (rows == 0) return ok();
  return hip_status(sxa::launch_combine(o_parts, part_dtype == SXA_BF16, lse_parts, n_parts, rows, d,
                                        o_out, out_dtype == SXA_BF16, lse_out,
                                        static_cast<hipStream_t>(stream)),
                    "lse_combine launch");
}

int chunk_cost(const int32_t* anchor, const int32_t* sample_start, int32_t n_blk,
               int32_t block_size, int32_t n_ctx, int32_t chunk_size, int64_t* cost_out,
               void* stream) {
  if (block_size != sxa::kBlock)
    return fail(SXA_EUNSUPPORTED, "block_size %d is not supported (only 16)", block_size);
  if (n_blk < 0 || n_ctx < 0) return fail(SXA_EINVAL, "n_blk and n_ctx must be >= 0");
  if (chunk_size <= 0) return fail(SXA_EINVAL, "chunk_size must be > 0 (got %d)", chunk_size);
  if (n_ctx > 0 && cost_out == nullptr) return fail(SXA_EINVAL, "cost_out must not be NULL");
  if (n_blk > 0 && (anchor == nullptr || sample_start == nullptr))
    return fail(SXA_EINVAL, "anchor and sample_start must not be NULL");
  const int64_t n_chunk = (static_cast<int64_t>(n_ctx) + chunk_size - 1) / chunk_size;
  if (n_chunk == 0) return ok();
  if (n_blk == 0) {
    return hip_status(sxa::launch_zero_words(cost_out, 2 * n_chunk, static_cast<hipStream_t>(stream)),
                      "chunk_cost zero fill");
  }
  return hip_status(sxa::launch_chunk_cost(anchor, sample_start, n_blk, n_ctx, chunk_size, cost_out,
                                           static_cast<hipStream_t>(stream)),
                    "chunk_cost launch");
}

int context_gather(const void* src, int64_t row_bytes, const int32_t* chunk_gstart,
                   const int32_t* chunk_len, int32_t n_chunk, int64_t n_dst_rows, void* dst,
                   void* stream) {
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(SXA_EINVAL, "row_bytes must be a positive multiple of 16 (got %lld)",
                static_cast<long long>(row_bytes));
  if (n_chunk < 0 || n_dst_rows < 0) return fail(SXA_EINVAL, "n_chunk and n_dst_rows must be >= 0");
  if (n_chunk > 0 && (chunk_gstart == nullptr || chunk_len == nullptr))
    return fail(SXA_EINVAL, "chunk_gstart and chunk_len must not be NULL");
  if (n_dst_rows > 0 && (src == nullptr || dst == nullptr)) return fail(SXA_EINVAL, "src and dst must not be NULL");
  if (n_chunk == 0 || n_dst_rows == 0) return ok();
  return hip_status(sxa::launch_context_gather(src, row_bytes, chunk_gstart, chunk_len, n_chunk, n_dst_rows,
                                               dst, static_cast<hipStream_t>(stream)),
                    "context_gather launch");
}

int lpt_assign(const int64_t* cost, int32_t n_chunk, int32_t n_bin, int32_t* bin_of_chunk,
               int64_t* bin_load) {
  if (n_bin <= 0) return fail(SXA_EINVAL, "n_bin must be > 0 (got %d)", n_bin);
  if (n_chunk <= 0 || n_chunk % n_bin != 0)
    return fail(SXA_EINVAL, "n_chunk (%d) must be a positive multiple of n_bin (%d)", n_chunk, n_bin);
  if (cost == nullptr || bin_of_chunk == nullptr || bin_load == nullptr)
    return fail(SXA_EINVAL, "cost, bin_of_chunk and bin_load must not be NULL");
  for (int32_t i = 0; i < n_chunk; ++i)
    if (cost[i] < 0) return fail(SXA_EINVAL, "cost[%d] is negative", i);
  sxa::lpt_assign_host(cost, n_chunk, n_bin, bin_of_chunk, bin_load);
  return ok();
}

int lpt_plan(const int64_t* cost, const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
             int32_t n_bin, int32_t* bin_of_chunk, int64_t* bin_load, int32_t* plan_gstart, int32_t* plan_len,
             void* stream) {
  if (n_bin <= 0) return fail(SXA_EINVAL, "n_bin must be > 0 (got %d)", n_bin);
  if (n_chunk <= 0 || n_chunk % n_bin != 0)
    return fail(SXA_EINVAL, "n_chunk (%d) must be a positive multiple of n_bin (%d)", n_chunk, n_bin);
  if (n_chunk > sxa::kMaxPlanChunks || n_bin > sxa::kMaxPlanBins)
    return fail(SXA_EUNSUPPORTED, "lpt_plan takes at most %d chunks and %d bins (got %d, %d; use lpt_assign)",
                sxa::kMaxPlanChunks, sxa::kMaxPlanBins, n_chunk, n_bin);
  if (cost == nullptr || chunk_gstart == nullptr || chunk_len == nullptr || bin_of_chunk == nullptr ||
      bin_load == nullptr || plan_gstart == nullptr || plan_len == nullptr)
    return fail(SXA_EINVAL, "lpt_plan: pointers must not be NULL");
  return hip_status(sxa::launch_lpt_plan(cost, n_chunk, n_bin, chunk_gstart, chunk_len, bin_of_chunk, bin_load,
                                         plan_gstart, plan_len, static_cast<hipStream_t>(stream)),
                    "lpt_plan launch");
}

}  // extern "C"
