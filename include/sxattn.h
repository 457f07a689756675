/*
 * sxattn.h - C ABI of libsxattn: anchor-masked block-sparse cross-attention
 * for one device's share of a packed context, on MI355X (gfx950).
 *
 * The operation is the one behind Split-KV context parallelism for training
 * diffusion drafters ("Split-KV speeds diffusion drafter training by keeping
 * long-context data local", arXiv 2611.05926):
 *   - anchors sampled inside each packed sample open blocks of draft tokens;
 *     every block attends to the preceding context of its own sample and to
 *     all tokens of its own block (section "Why short queries change the
 *     problem");
 *   - keys/values stay local; every query is evaluated against the local
 *     chunks and the partial results carry normalisation statistics from
 *     which they are merged exactly (section "Exchange the smaller side");
 *   - each context chunk gets a cost from its realised attention usage and a
 *     longest-processing-time-first planner balances chunks across devices
 *     with equal chunk counts (section "Balance actual attention work").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Block size B is 16 draft tokens.  n_q = n_blk * B queries.
 * Device tensors are caller-owned, contiguous, token-major:
 *   q, o, dout, dq_accum : [n_q][hq][d]
 *   k, v, dk, dv          : [n_loc][hkv][d]   local rows = the listed chunks back to back
 *   k_self, v_self, dk_self, dv_self : [n_q][hkv][d]  keys/values of the draft tokens
 *   (gradients are float32; dk, dv, dk_self, dv_self may be bf16, see sparse_xattn_bwd)
 *   lse                   : [n_q][hq] float32
 *   delta_ws              : [2][n_q][hq] float32
 * Query head h reads kv head h / (hq / hkv).
 * Metadata (device int32 arrays):
 *   anchor[b], sample_start[b]  global packed positions of block b's anchor and of
 *                               the start of its sample; block b may attend to
 *                               context positions j with sample_start[b] <= j < anchor[b]
 *                               (the anchor itself is excluded);
 *   chunk_gstart[i], chunk_len[i]  chunk i of the local buffer holds global positions
 *                               [chunk_gstart[i], chunk_gstart[i] + chunk_len[i]).
 * The own-block term: query i of block b also attends to rows b*B .. b*B+B-1 of
 * k_self/v_self (all of them, no causal order).  Pass k_self/v_self on exactly one
 * call per pass (forward or backward) and NULL on the others.
 * Logits are scale * <q, k> (scale is a float32 value, usually 1/sqrt(d)); lse is the
 * natural-log log-sum-exp of the scaled logits.  A row with no allowed key in a call
 * gets lse = -inf and o = 0.
 *
 * Streams and ownership: `stream` is a hipStream_t (NULL = the default stream).
 * Device work is enqueued asynchronously; outputs are valid after the stream is
 * synchronised.  The library allocates no device memory; scratch is passed in.
 *
 * Errors: every call returns an sxa_status.  Arguments are validated on the host
 * before anything is enqueued (null pointers, sizes, dtypes, head counts); on a
 * validation error nothing is launched and outputs are untouched.  A failed launch
 * returns SXA_EHIP.  sxa_last_error() gives a message for the last failure of the
 * calling thread.  Metadata values on the device are not validated: anchors must
 * satisfy sample_start <= anchor, chunks must not overlap, and chunk lengths must
 * sum to n_loc; other values give unspecified (but in-bounds) results.
 */
#ifndef SXATTN_H
#define SXATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SXA_F32 = 0, SXA_BF16 = 1 } sxa_dtype;

typedef enum {
  SXA_OK = 0,
  SXA_EINVAL = -1,        /* bad argument (null pointer, size, dtype, divisibility) */
  SXA_EUNSUPPORTED = -2,  /* valid but not implemented (head_dim, block size, dtype pair) */
  SXA_EHIP = -3           /* a HIP runtime call or kernel launch failed */
} sxa_status;

/*
 * Partial forward over this call's local chunks (plus the own-block term if
 * k_self != NULL).  Follows "Why short queries change the problem" (mask) and
 * "Exchange the smaller side" (local keys/values, partial output with
 * statistics).
 *   q [n_q][hq][d], k/v [n_loc][hkv][d] in in_dtype; d in {64, 128}; block_size == 16;
 *   hq % hkv == 0.  n_chunk >= 0 (0 with k_self set gives the own-block partial alone).
 *   Size limits (SXA_EUNSUPPORTED beyond them): n_blk * 16 * hq < 2^29, hkv <= 4096.
 *   o [n_q][hq][d] in o_dtype (SXA_F32 or SXA_BF16; SXA_F32 input requires SXA_F32 output),
 *   lse [n_q][hq] float32.  Both are overwritten.
 *   workspace, workspace_bytes: optional device scratch (at least
 *   sparse_xattn_fwd_workspace_bytes() bytes, else ignored).  With it the bf16 path
 *   first ranks its query row groups by the number of key tiles they read and
 *   dispatches the heaviest first; results do not depend on it.  With at least
 *   sparse_xattn_fwd_split_workspace_bytes() bytes the bf16 path also splits the key
 *   tiles of every row group that reads more than 1.5 times the mean work of a
 *   compute unit into pieces run by separate workgroups, whose partial O and lse a merge pass
 *   combines exactly as lse_combine does ("Exchange the smaller side": partials with
 *   their statistics merge into the unsplit result).  Results then agree with the
 *   unsplit call up to float32 rounding, not bit for bit.  Calls that share a
 *   workspace must be ordered on one stream.
 * bf16 inputs run on bf16 MFMA with float32 accumulation and statistics; float32
 * inputs run in float32 throughout.
 */
int sparse_xattn_fwd(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                     int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                     float scale, const int32_t* anchor, const int32_t* sample_start,
                     const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                     int64_t n_loc, const void* k_self, const void* v_self,
                     void* o, sxa_dtype o_dtype, float* lse, void* workspace,
                     int64_t workspace_bytes, void* stream);

/*
 * sparse_xattn_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors are those of sparse_xattn_fwd
 * called with a workspace of sparse_xattn_fwd_workspace_bytes() bytes: the bf16 path
 * ranks its query row groups and dispatches the heaviest first (no split schedule),
 * with the ranking kept in a library-owned static device array of 4096 int32 (16 KiB)
 * that every device running the library holds until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine); the caller still
 * passes inputs and outputs.  Beyond 4096 row groups of 256 query rows per kv head
 * (n_blk * 16 * hq / hkv > 1048576) it returns SXA_EUNSUPPORTED before anything is
 * enqueued.  Every call on one device uses that device's array, which keeps the last
 * call's contents (nothing in it needs clearing: each call rewrites what it reads);
 * calls that overlap on one device (concurrent streams or threads) race on it and
 * must be ordered by the caller.
 */
int sparse_xattn_fwd_noalloc(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                             int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                             float scale, const int32_t* anchor, const int32_t* sample_start,
                             const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                             int64_t n_loc, const void* k_self, const void* v_self, void* o,
                             sxa_dtype o_dtype, float* lse, void* stream);

/* Workspace bytes of sparse_xattn_fwd's load balancing (0 for invalid sizes). */
int64_t sparse_xattn_fwd_workspace_bytes(int32_t n_blk, int32_t hq, int32_t hkv);

/* Workspace bytes of sparse_xattn_fwd's split schedule (above) on the current device:
 * the plan, and float32 partial O and lse for up to 2 * (compute units) pieces of 256
 * query rows (about 67 MB at d = 128 on 256 compute units).  0 for invalid sizes and
 * beyond 4096 row groups of 256 query rows per kv head, where no split is done. */
int64_t sparse_xattn_fwd_split_workspace_bytes(int32_t n_blk, int32_t hq, int32_t hkv, int32_t d);

/* Phases of sparse_xattn_bwd (bit flags; naming none of DELTA, DQ, DKDV means all
 * three) and their modifiers. */
enum {
  SXA_BWD_DELTA = 1,         /* pre-pass: delta_ws = (rowsum(dout * o), lse * log2 e) */
  SXA_BWD_DQ = 2,            /* add this call's query gradient to dq_accum */
  SXA_BWD_DKDV = 4,          /* write dk, dv (and dk_self, dv_self) */
  SXA_BWD_DQ_OVERWRITE = 8,  /* with SXA_BWD_DQ: overwrite dq_accum instead of adding */
  SXA_BWD_DKDV_BF16 = 16     /* with SXA_BWD_DKDV: dk, dv, dk_self, dv_self are bf16 */
};

/*
 * Backward of this call's chunks (and own-block term if k_self != NULL), from the
 * merged output o, merged lse and upstream gradient dout (all [n_q][hq], dtype
 * in_dtype for o/dout).  Keys/values stay local: the gradient of the local rows is
 * produced here ("Exchange the smaller side": local in forward and backward).
 *   delta_ws [2][n_q][hq] float32: written by the SXA_BWD_DELTA phase, read by the
 *            others: plane 0 holds rowsum(dout * o), plane 1 lse * log2(e) (+inf
 *            where lse = -inf).  A caller that already holds it from an earlier call
 *            with the same o, dout and lse may skip the phase.
 *   dq_accum [n_q][hq][d] float32: this call's query gradient is ADDED to it (or
 *            written, with SXA_BWD_DQ_OVERWRITE), so per-chunk calls accumulate.
 *   dk, dv   [n_loc][hkv][d] float32 (bf16 with SXA_BWD_DKDV_BF16, bf16 inputs
 *            only): overwritten.  The sums are formed in float32 either way; the
 *            bf16 form rounds each final value to nearest even.
 *   dk_self, dv_self [n_q][hkv][d] float32 (bf16 with SXA_BWD_DKDV_BF16): overwritten
 *            when k_self != NULL (must then be non-NULL), ignored otherwise.
 *   workspace, workspace_bytes: optional device scratch for the bf16 dK/dV phase.
 *            With at least sparse_xattn_bwd_workspace_bytes() bytes the phase is
 *            load-balanced: one workgroup per compute unit, each taking an equal
 *            share of all (key tile, query step) work, with the partial sums of
 *            tiles split between workgroups added by a second pass.  With NULL (or
 *            too small) every 256-key tile is handled by one workgroup.  With at
 *            least sparse_xattn_bwd_split_workspace_bytes() bytes the bf16 dQ phase
 *            also runs the split schedule of sparse_xattn_fwd: query row groups that
 *            read more than 1.5 times the mean work of a compute unit are cut into
 *            pieces of their key tiles, each piece's dQ sum goes to a slot, and a
 *            second pass adds the pieces to dq_accum (dQ is a plain sum over keys,
 *            "Exchange the smaller side"); results then agree with the unsplit phase
 *            up to float32 summation order.  Contents are scratch; calls that share
 *            a workspace must be ordered on one stream.
 *   flags    SXA_BWD_* bits selecting the phases; they run in the order
 *            DELTA, DQ, DKDV on `stream`.
 */
int sparse_xattn_bwd(const void* q, const void* k, const void* v, sxa_dtype in_dtype,
                     int32_t n_blk, int32_t block_size, int32_t hq, int32_t hkv, int32_t d,
                     float scale, const int32_t* anchor, const int32_t* sample_start,
                     const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
                     int64_t n_loc, const void* k_self, const void* v_self,
                     const void* o, const void* dout, const float* lse,
                     float* delta_ws, float* dq_accum, void* dk, void* dv,
                     void* dk_self, void* dv_self, void* workspace, int64_t workspace_bytes,
                     int32_t flags, void* stream);

/* Workspace bytes for the load-balanced dQ and dK/dV phases of sparse_xattn_bwd on
 * the current device (a function of the sizes and the device's compute-unit count;
 * 0 for invalid sizes). */
int64_t sparse_xattn_bwd_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv,
                                         int32_t d);

/* Workspace bytes for the same phases with the split dQ schedule (above) on the
 * current device: sparse_xattn_bwd_workspace_bytes() rounded up to 256, plus the plan
 * and float32 slots of up to 2 * (compute units) pieces of 256 query rows.  0 for
 * invalid sizes and beyond 4096 row groups of 256 query rows per kv head. */
int64_t sparse_xattn_bwd_split_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv,
                                               int32_t d);

/*
 * Exact merge of n_parts partials from their log-sum-exp statistics
 * ("Exchange the smaller side": partial results are combined from normalisation
 * statistics so that the original attention is reconstructed exactly).
 *   o_parts [n_parts][rows][d] in part_dtype, lse_parts [n_parts][rows] float32
 *   (rows = n_q * hq for attention partials).  A partial with lse = -inf is skipped
 *   and its o rows are not read.
 *   o_out [rows][d] in out_dtype, lse_out [rows] float32: overwritten with
 *   lse = m + ln(sum_p exp(lse_p - m)), o = sum_p exp(lse_p - lse) o_p; rows whose
 *   partials are all empty get lse = -inf, o = 0.  d must be 64, 128 or 256.
 */
int lse_combine(const void* o_parts, sxa_dtype part_dtype, const float* lse_parts,
                int32_t n_parts, int64_t rows, int32_t d, void* o_out, sxa_dtype out_dtype,
                float* lse_out, void* stream);

/*
 * Realised attention cost of every contiguous context chunk
 * ("Balance actual attention work": a chunk is priced by the attention work that
 * lands on it, which any device can count from the metadata of all query blocks).
 *   cost_out[c] (device int64, c < ceil(n_ctx / chunk_size)) = number of
 *   (query token, key) pairs with the key in [c*chunk_size, min((c+1)*chunk_size, n_ctx))
 *   allowed by the anchor mask, for one head; own-block pairs are not counted.
 *   Exact integer result.
 */
int chunk_cost(const int32_t* anchor, const int32_t* sample_start, int32_t n_blk,
               int32_t block_size, int32_t n_ctx, int32_t chunk_size, int64_t* cost_out,
               void* stream);

/*
 * Longest-processing-time-first assignment of chunks to n_bin devices with equal
 * chunk counts ("Balance actual attention work").  HOST pointers, synchronous.
 *   cost[n_chunk] int64 >= 0; n_chunk must be a positive multiple of n_bin.
 *   Chunks are taken by (cost descending, index ascending); each goes to the bin
 *   with the smallest (load, bin index) among bins holding fewer than n_chunk/n_bin
 *   chunks.  bin_of_chunk[n_chunk] and bin_load[n_bin] are overwritten.
 */
int lpt_assign(const int64_t* cost, int32_t n_chunk, int32_t n_bin, int32_t* bin_of_chunk,
               int64_t* bin_load);

/*
 * The same plan on the device ("Balance actual attention work"), so that a step that
 * prices its chunks on the GPU plans them without a round trip through the host.
 * DEVICE pointers, asynchronous on `stream`; one workgroup.
 *   cost[n_chunk] int64 >= 0 (not validated on the device); chunk_gstart[n_chunk],
 *   chunk_len[n_chunk] int32: each chunk's global start and length.
 *   bin_of_chunk[n_chunk] and bin_load[n_bin] are overwritten with exactly what
 *   lpt_assign returns for the same costs.  plan_gstart and plan_len
 *   [n_bin][n_chunk / n_bin] are overwritten with each bin's chunks (their global
 *   starts and lengths) in increasing chunk index: the chunk lists that
 *   context_gather and the attention calls of that bin take.
 *   n_chunk must be a positive multiple of n_bin (SXA_EINVAL); at most 4096 chunks
 *   and 1024 bins (SXA_EUNSUPPORTED beyond: use lpt_assign).
 */
int lpt_plan(const int64_t* cost, const int32_t* chunk_gstart, const int32_t* chunk_len, int32_t n_chunk,
             int32_t n_bin, int32_t* bin_of_chunk, int64_t* bin_load, int32_t* plan_gstart, int32_t* plan_len,
             void* stream);

/*
 * Context redistribution: copy the rows of the listed chunks of a packed context
 * tensor back to back into a device's local buffer ("Balance actual attention
 * work": after planning, context chunks are moved once per step to the device
 * that owns them).
 *   src [n_src_rows][row_bytes] device; chunk i covers src rows
 *   [chunk_gstart[i], chunk_gstart[i] + chunk_len[i]) (device int32 arrays);
 *   dst [sum chunk_len][row_bytes] device, overwritten.  row_bytes must be a
 *   multiple of 16; chunks must lie inside src (not validated on the device).
 */
int context_gather(const void* src, int64_t row_bytes, const int32_t* chunk_gstart,
                   const int32_t* chunk_len, int32_t n_chunk, int64_t n_dst_rows, void* dst,
                   void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* sxa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SXATTN_H */
