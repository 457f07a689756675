// Internal interface between the C-ABI host layer (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sxattn.h"

namespace sxa {

constexpr int kBlock = 16;  // draft tokens per anchor block

// Everything an attention launch needs; pointers are device pointers.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* k_self;  // nullable
  const void* v_self;
  int32_t n_blk, hq, hkv, d;
  float scale;
  const int32_t* anchor;
  const int32_t* sample_start;
  const int32_t* chunk_gstart;
  const int32_t* chunk_len;
  int32_t n_chunk;
  int64_t n_loc;
  // forward outputs
  void* o;
  bool o_bf16;
  float* lse;
  // backward inputs / outputs
  const void* o_in;
  const void* dout;
  const float* lse_in;
  float* delta;
  float* dq;
  void* dk;
  void* dv;
  void* dk_self;
  void* dv_self;
  int32_t flags;  // SXA_BWD_* phases (never 0 here)
  void* workspace;  // optional dK/dV split scratch (nullptr: no split)
  int64_t workspace_bytes;
  int32_t* rg_order;  // optional scratch for the row-group dispatch order (nullptr: index order)
  void* row_split;    // optional scratch of the split forward or dQ phase (nullptr: one workgroup per row group)
  int32_t n_cu;       // compute units of the device (used with row_split)
};

// Query rows per forward / dQ workgroup, and the largest row-group count that is
// dispatched in cost order (beyond it: index order).
constexpr int kRowsPerGroup = 256;
constexpr int kMaxOrderedGroups = 4096;
int64_t row_groups(const AttnArgs& a, int rows_per_group);
// Compute units of the current device (cached per device).
int n_compute_units();
// Write the row groups of `a` into order[0 .. n), most 64-key tiles first (no-op
// when there are more than kMaxOrderedGroups groups).
hipError_t launch_row_group_order(const AttnArgs& a, int rows_per_group, int32_t* order, hipStream_t s);

// Split schedule of the forward and of the dQ phase: a row group whose key tiles
// exceed the cap (1.5 times the mean tiles per compute unit, at least kMinSplitTiles)
// runs as equal pieces of its tile walk, each on its own workgroup; the pieces'
// partial results go to slots, and a merge pass writes the group's rows.  The plan
// lives in the caller's scratch:
struct RowSplit {
  int4* jobs;       // [n_groups + max_pieces]: {row group, first tile, end tile, slot or -1},
                    // most tiles first; row group -1: no job
  int4* groups;     // [max_pieces / 2]: {row group, first slot, pieces, 0}; row group -1: none
  float* part_lse;  // [max_pieces][hkv][kRowsPerGroup] forward: natural-log lse of each piece
  float* part_o;    // [max_pieces][hkv][kRowsPerGroup][d] forward: normalised partial O;
                    // dQ phase: the piece's scaled dQ sum
  int32_t max_pieces;
  int32_t max_extra;  // jobs beyond one per row group, per kv head (the grid's spare slots)
};
constexpr int kMinSplitTiles = 16;
// Pieces of split row groups per kv head: the cap is above the mean tiles per compute
// unit, so they never exceed 2 n_cu / hkv.
int32_t row_split_max_pieces(int32_t hkv, int32_t n_cu);
// Jobs a split adds (a group of T > cap tiles becomes ceil(T / cap) < T / cap + 1
// jobs, and the tiles of all groups sum to at most cap * 2 n_cu / (3 hkv)), so at most
// ceil(2 n_cu / (3 hkv)) per kv head; the grid carries that many spare job slots.
int32_t row_split_max_extra(int32_t hkv, int32_t n_cu);
// Bytes of the split forward's scratch (0 if not representable or beyond the
// ordered-group limit).
int64_t row_split_bytes(int32_t n_blk, int32_t hq, int32_t hkv, int32_t d, int32_t n_cu);
RowSplit row_split_layout(void* ws, const AttnArgs& a);
// The plan of the split forward into sp (one workgroup).
hipError_t launch_row_split_plan(const AttnArgs& a, const RowSplit& sp, hipStream_t s);

// Bytes of dK/dV split scratch for n_loc local rows (0 if not representable).
int64_t bwd_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv, int32_t d);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_fwd_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_delta(const AttnArgs& a, bool bf16, hipStream_t s);
hipError_t launch_combine(const void* o_parts, bool part_bf16, const float* lse_parts,
                          int32_t n_parts, int64_t rows, int32_t d, void* o_out, bool out_bf16,
                          float* lse_out, hipStream_t s);
// Zero n_words 32-bit words with a fill kernel (no hipMemsetAsync, so the call is
// safe inside a captured graph).
hipError_t launch_zero_words(void* p, int64_t n_words, hipStream_t s);
hipError_t launch_context_gather(const void* src, int64_t row_bytes, const int32_t* chunk_gstart,
                                 const int32_t* chunk_len, int32_t n_chunk, int64_t n_dst_rows,
                                 void* dst, hipStream_t s);
hipError_t launch_chunk_cost(const int32_t* anchor, const int32_t* sample_start, int32_t n_blk,
                             int32_t n_ctx, int32_t chunk_size, int64_t* cost, hipStream_t s);
// The device LPT plan (one workgroup; the arrays live in LDS up to these sizes).
constexpr int kMaxPlanChunks = 4096;
constexpr int kMaxPlanBins = 1024;
hipError_t launch_lpt_plan(const int64_t* cost, int32_t n_chunk, int32_t n_bin, const int32_t* chunk_gstart,
                           const int32_t* chunk_len, int32_t* bin_of, int64_t* bin_load, int32_t* plan_gstart,
                           int32_t* plan_len, hipStream_t s);

}  // namespace sxa
