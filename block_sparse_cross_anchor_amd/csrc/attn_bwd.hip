// bf16 backward of the anchor-masked block-sparse cross-attention on gfx950 MFMA.
//
// Split-KV keeps keys and values local in the backward pass as well ("Split-KV
// speeds diffusion drafter training...", section "Exchange the smaller side"):
// each call produces the gradient of its local key/value rows and adds its share
// of the query gradient.  The probabilities are recomputed from the merged
// log-sum-exp, so no forward state is needed beyond the merged O and lse:
//   P = exp(scale q.k - lse),  delta = rowsum(dO * O),  dS = P * (dO.v - delta)
//   dQ += scale dS K,  dK = scale dS^T Q,  dV = P^T dO   (dK, dV summed over the
//   query heads that share a kv head).
//
// Two kernels, neither needs atomics:
//   * dq kernel (query-major, same decomposition as the forward): each wave owns
//     32 query rows and walks its allowed key tiles; per 64-key tile it recomputes
//     S^T = K Q^T and dP^T = V dO^T, forms dS^T in registers and accumulates
//     dQ^T += K^T dS^T (K staged row-major and transposed in LDS, V row-major).
//   * dkdv kernel (key-major): each wave owns 32 keys (K, V held in registers as
//     MFMA operands) and walks the 32-row query steps whose blocks can read them;
//     per step it computes S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//     dK^T += Q^T dS (Q and dO staged row-major and transposed in LDS).
// The recomputation of S and dP in both kernels is the price of avoiding
// cross-workgroup reductions of dQ.
#include "device_common.h"
#include "internal.h"
#include "kv_walk.h"
#include "lds_tile.h"

namespace sxa {
namespace {

#ifndef SXA_DQ_WAVES
#define SXA_DQ_WAVES 8
#endif
#ifndef SXA_KV_HALVES
#define SXA_KV_HALVES 1
#endif
constexpr int kDqWaves = SXA_DQ_WAVES;  // waves per dq workgroup (32 query rows each)
constexpr int kKvHalves = SXA_KV_HALVES;    // 32-key halves per dkdv wave
constexpr int kKvWaves = 8 / kKvHalves;      // waves per dkdv workgroup (256 keys)

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_self;
  const uint16_t* v_self;
  const uint16_t* dout;
  const float* lse;
  const float* delta;  // [2][n_q][hq]: delta rows, then lse * log2(e) (+inf where lse = -inf)
  float* dq;
  void* dk;  // float32, or bf16 with grad_bf16
  void* dv;
  void* dk_self;
  void* dv_self;
  const int32_t* anchor;
  const int32_t* sample_start;
  const int32_t* chunk_gstart;
  const int32_t* chunk_len;
  int64_t n_loc;
  int32_t n_blk, hq, hkv, n_chunk;
  float scale;
  float scale_log2;  // scale * log2(e)
  int32_t dq_overwrite;
  int32_t grad_bf16;  // dK, dV (and own-block) written as bf16, rounded to nearest even
  const int32_t* rg_order;  // dQ: row group of workgroup blockIdx / hkv (nullptr: identity)
  // split dQ (jobs != nullptr): job blockIdx / hkv = {row group, first tile, end tile,
  // slot}; a job with a slot writes its scaled dQ sum there instead of adding it
  const int4* jobs;
  float* part_dq;
};

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// Four gradient values to element offset `o` of a float32 or bf16 gradient tensor.
__device__ __forceinline__ void store_grad4(void* base, int64_t o, const f32x4& x, bool bf16) {
  if (bf16)
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + o) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  else
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + o) = x;
}

// ============================================================================ dq kernel
//
// Query-major, same tiles as the forward: a workgroup of kDqWaves waves owns 256
// query rows of one kv head (32 per wave, Q and dO held in registers as MFMA B
// operands) and walks the 64-key tiles their blocks may read (kv_walk.h), copied
// into LDS three tiles deep.  Per tile: S^T = K Q^T, dP^T = V dO^T, dS^T in
// registers, dQ^T += K^T dS^T (K^T from the transposing read of the K tile).

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kDqWaves, 64 * kDqWaves))) void dq_bf16_kernel(
    BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int ROWS = 32 * kDqWaves;
  using Dma = TileDma<D, kDqWaves, true>;
  __shared__ __attribute__((aligned(256))) uint16_t bufs[3][Dma::ELEMS];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  const int g = blockIdx.x % p.hkv;
  int wg, t_skip = 0, t_left = 0x7fffffff;
  if (p.jobs) {
    const int4 jb = p.jobs[blockIdx.x / p.hkv];
    if (jb.x < 0) return;  // more job slots than jobs
    wg = __builtin_amdgcn_readfirstlane(jb.x);  // uniform: kept in scalar registers
    t_skip = __builtin_amdgcn_readfirstlane(jb.y);
    t_left = __builtin_amdgcn_readfirstlane(jb.z - jb.y);
  } else {
    wg = p.rg_order ? p.rg_order[blockIdx.x / p.hkv] : static_cast<int>(blockIdx.x / p.hkv);
  }
  const int grp = p.hq / p.hkv;
  const int64_t n_q = static_cast<int64_t>(p.n_blk) * kBlock;
  const int64_t R = n_q * grp;
  const int64_t wg_row0 = static_cast<int64_t>(wg) * ROWS;
  const int64_t wg_last = min(wg_row0 + ROWS - 1, R - 1);
  const int b_first = static_cast<int>(wg_row0 / grp / kBlock);
  const int b_last = static_cast<int>(wg_last / grp / kBlock);
  int LO = 0x7fffffff, HI = -0x7fffffff;
  for (int b = b_first; b <= b_last; ++b) {
    LO = min(LO, p.sample_start[b]);
    HI = max(HI, p.anchor[b]);
  }
  Walk w;
  w.start(p.k_self != nullptr, b_first, b_last);
  // a piece of a split row group: skip to its first tile, stop after its last
  Tile skipped;
  for (int i = 0; i < t_skip; ++i) walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, skipped);
  auto next_tile = [&](Tile& t) {
    if (t_left == 0) return false;
    --t_left;
    return walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, t);
  };
  Tile cur;
  const bool have = next_tile(cur);

  // this lane's query row (column of the 32-row N tile)
  const int64_t r = wg_row0 + 32 * wave + l32;
  const bool valid = r < R;
  const int64_t rr = valid ? r : 0;
  const int64_t tok = rr / grp;
  const int hh = static_cast<int>(rr % grp);
  const int blk = static_cast<int>(tok / kBlock);
  const int64_t orow = tok * p.hq + static_cast<int64_t>(g) * grp + hh;
  if (!have) {  // no key of this call reaches these rows: nothing to add
    const int slot = p.jobs ? p.jobs[blockIdx.x / p.hkv].w : -1;  // re-read: not held in registers
    if (slot >= 0) {  // (a piece always has tiles; an empty one adds zeros)
      const int64_t pr = (static_cast<int64_t>(slot) * p.hkv + g) * ROWS + 32 * wave + l32;
#pragma unroll
      for (int d0 = h2 * (D / 2); d0 < (h2 + 1) * (D / 2); d0 += 4)
        *reinterpret_cast<f32x4*>(p.part_dq + pr * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (p.dq_overwrite && valid) {
      // the two lanes of a row (h2 = 0, 1) each clear half of it
#pragma unroll
      for (int d0 = h2 * (D / 2); d0 < (h2 + 1) * (D / 2); d0 += 4)
        *reinterpret_cast<f32x4*>(p.dq + orow * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int clo = valid ? p.sample_start[blk] : 0, chi = valid ? p.anchor[blk] : 0;
  const int slo = valid ? kBlock * blk : 0, shi = valid ? kBlock * blk + kBlock : 0;
  // lse in log2 units (+inf for rows without keys: exp2(x - inf) = 0), and delta
  const float lse2 = valid ? p.delta[n_q * p.hq + orow] : INFINITY;
  const float dlt = p.delta[orow];
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p.q + orow * D + 16 * ks + 8 * h2));
    df[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p.dout + orow * D + 16 * ks + 8 * h2));
  }

  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[dt][i] = 0.f;

  // LDS byte offsets within a tile buffer (see LdsTile): K / V rows 32 mt + l32,
  // transposed K reads of the key steps
  int f_k = LdsTile<D>::frag_off(l32, h2);
  int t_a = LdsTile<D>::tr_off(4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
  int t_b = LdsTile<D>::tr_off(8 + 4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
  constexpr uint32_t kVOff = kTileKeys * D * 2;  // V rows follow the K rows

  // Three-stage pipeline: tile t is computed from buffer t % 3 while the copies of
  // tiles t + 1 and t + 2 are in flight.  The prologue's own loads complete first,
  // so that the only vector-memory operations in flight in the loop are the copies.
  wait_vmcnt<0>();
  Tile n1, n2;
  const Dma dma(p.hkv, wave, lane);
  dma.issue(cur, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[0]));
  bool have1 = next_tile(n1);
  if (have1) dma.issue(n1, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[1]));
  int cb = 0;
  while (true) {
    if (have1) wait_vmcnt<Dma::NI>();  // this wave's copies of `cur` landed (n1 may fly)
    else wait_vmcnt<0>();
    barrier_nofence();                 // ... and every wave's; all reads of the third buffer are done
    const bool have2 = next_tile(n2);  // false once exhausted
    if (have2) dma.issue(n2, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[cb == 0 ? 2 : cb - 1]));

    // per-lane constants are redefined opaquely per tile so that derived addresses
    // are recomputed rather than held
    asm volatile("" : "+v"(f_k), "+v"(t_a), "+v"(t_b));
    const int lo = cur.self ? slo : clo, hi = cur.self ? shi : chi;
    const int a_lo = max(lo - cur.coord0, 0), a_hi = min(hi - cur.coord0, cur.nrows);
    const bool any = a_lo < a_hi;
    const bool full = (a_lo == 0) & (a_hi == kTileKeys);
    if (__any(any)) {
      const bool all_full = __all(full);
      const uint32_t base = lds_addr(bufs[cb]);
      const uint32_t kb = base + f_k, ta = base + t_a, tb = base + t_b;
      // The tile's two 32-key halves one after the other: S^T and dP^T of half mt
      // (16 MFMAs), its dS^T (VALU), then the dQ^T MFMAs of its two 16-key steps.
      // Only one half's S^T, dP^T accumulators are live at a time, which leaves the
      // registers for reading every LDS fragment one MFMA pair ahead of its use; and
      // the exponent of half 0 has half 1's MFMAs to overlap with.
      bf16x8 kf = lds_frag(kb), vf = lds_frag(kb + kVOff);
      bf16x8 kt = lds_frag_t(ta, tb);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ck = kf, cv = vf;
          const int nx = mt * KS + ks + 1;  // next (half, k-step)
          if (nx < 2 * KS) {
            const uint32_t o = (kb ^ (32 * (nx % KS))) + (nx / KS) * 64 * D;
            kf = lds_frag(o);
            vf = lds_frag(o + kVOff);
          }
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ck, qf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv, df[ks], pacc, 0, 0, 0);
        }
        // exponent in place; keys outside the row's interval get exp2(-inf) = 0
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(sacc[i], p.scale_log2, -lse2);
        if (!all_full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * mt + 8 * (i / 4) + 4 * h2 + (i % 4);
            if (key < a_lo || key >= a_hi) sacc[i] = -INFINITY;
          }
        }
        u32x4 dsw[2];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float d0 = __builtin_amdgcn_exp2f(sacc[2 * q]) * (pacc[2 * q] - dlt);
          const float d1 = __builtin_amdgcn_exp2f(sacc[2 * q + 1]) * (pacc[2 * q + 1] - dlt);
          dsw[q / 4][q % 4] = pack_bf16x2(d0, d1);
        }
#pragma unroll
        for (int j = 0; j < 2 * DT; ++j) {
          const int kq = 2 * mt + j / DT, dt = j % DT;
          const bf16x8 ck = kt;
          const int nx = 2 * DT * mt + j + 1;  // next (16-key step, d tile)
          if (nx < 4 * DT) {
            const int kq1 = nx / DT, dt1 = nx % DT;
            kt = lds_frag_t((ta ^ (64 * dt1)) + kq1 * 32 * D, (tb ^ (64 * dt1)) + kq1 * 32 * D);
          }
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ck, __builtin_bit_cast(bf16x8, dsw[kq % 2]),
                                                              dqacc[dt], 0, 0, 0);
        }
      }
    }
    if (!have1) break;
    cur = n1;
    n1 = n2;
    have1 = have2;
    cb = cb == 2 ? 0 : cb + 1;
  }

  if (!valid) return;
  const int slot = p.jobs ? p.jobs[blockIdx.x / p.hkv].w : -1;  // re-read: not held in registers
  if (slot >= 0) {  // a piece: its scaled sum to the slot (the merge adds the pieces)
    const int64_t pr = (static_cast<int64_t>(slot) * p.hkv + g) * ROWS + 32 * wave + l32;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = p.scale * dqacc[dt][4 * jj + i];
        *reinterpret_cast<f32x4*>(p.part_dq + pr * D + 32 * dt + 8 * jj + 4 * h2) = acc;
      }
    return;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float* dst = p.dq + orow * D + 32 * dt + 8 * jj + 4 * h2;
      f32x4 acc = p.dq_overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(dst);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(p.scale, dqacc[dt][4 * jj + i], acc[i]);
      *reinterpret_cast<f32x4*>(dst) = acc;
    }
}

// Merge of the split row groups' dQ pieces, one workgroup per (kv head, run of
// 256 / (d / 4) rows) looping over the split groups until the first unused entry,
// d / 4 lanes per row: dq = (overwrite ? 0 : dq) + the pieces' sums in piece order.
// A small fixed grid, as for the forward's merge.
template <int D>
__global__ __launch_bounds__(256) void dq_merge_kernel(RowSplit sp, float* dq, int32_t n_blk, int32_t hq, int32_t hkv,
                                                       int32_t overwrite) {
  constexpr int LPR = D / 4;                 // lanes per row, 4 values each
  constexpr int RPW = 256 / LPR;             // rows per workgroup
  const int g = blockIdx.x % hkv;
  const int run = blockIdx.x / hkv;  // < kRowsPerGroup / RPW
  const int grp = hq / hkv;
  const int64_t R = static_cast<int64_t>(n_blk) * kBlock * grp;
  const int sub = threadIdx.x % LPR;
  const int lr = run * RPW + threadIdx.x / LPR;
  for (int sg = 0; sg < sp.max_pieces / 2; ++sg) {
    const int4 jb = sp.groups[sg];
    if (jb.x < 0) break;  // used entries come first
    const int64_t r = static_cast<int64_t>(jb.x) * kRowsPerGroup + lr;
    if (r >= R) continue;
    const int64_t orow = (r / grp) * hq + static_cast<int64_t>(g) * grp + static_cast<int>(r % grp);
    f32x4* dst = reinterpret_cast<f32x4*>(dq + orow * D + 4 * sub);
    f32x4 acc = overwrite ? f32x4{0.f, 0.f, 0.f, 0.f} : *dst;
    for (int k = 0; k < jb.z; ++k)
      acc += *reinterpret_cast<const f32x4*>(
          sp.part_o + ((static_cast<int64_t>(jb.y + k) * hkv + g) * kRowsPerGroup + lr) * D + 4 * sub);
    *dst = acc;
  }
}

// ============================================================================ dkdv kernel
//
// Key-major.  A workgroup of kKvWaves waves handles 32 keys per wave, i.e. a "key
// tile" of 256 consecutive key rows of one kv head (local context rows, or own-block
// rows for the tiles after the context ones).  K of a wave's keys is held in
// registers (MFMA B operand of S = Q K^T); V of the tile sits in LDS (B operand of
// dP = dO V^T).
//
// Query side.  The grp query heads of kv head g are visited in "steps" of 32 query
// rows that start on a token boundary: ts = 32 / grp whole tokens with all their
// heads when grp <= 32 (rows past ts grp are padding), or 32 heads of one token when
// grp > 32.  Row i of a step is token tok0 + i / gs, head h0 + i % gs of the group
// (gs = min(grp, 32)), so every lane copies from a fixed offset to the step's first
// element.  A step covers at most 32 tokens and starts on a multiple of ts, so it
// meets at most two 16-token blocks; its mask is two key intervals split at a row.
// A step "hits" a tile when one of its blocks' intervals meets the tile's
// key-coordinate range (own-block tiles: when it holds one of their blocks).
//
// Schedule.  The work is the list of (kv head, tile, hit step) triples, and a key
// tile near the start of a long sample is hit by many times more steps than the
// average one.  With a workspace, a count pass gives every tile its number of hit
// steps and their list in order (a segment's steps are then read from the list, not
// found by scanning every step of the kv head), and the kernel runs one workgroup
// per compute unit, each taking an equal
// contiguous share of the list ("stream-K"): inside a share only the first and the
// last tile can be partial; their fp32 sums go to the share's two workspace slots and
// a reduce pass adds the slots of each such tile.  Tiles a share covers whole are
// written directly.  Without a workspace every (tile, kv head) gets one workgroup.
//
// Pipeline.  The Q and dO rows of a step, and its per-row lse and delta, are copied
// from HBM straight into LDS (global_load_lds), three steps deep: while step i is
// computed the copies of steps i+1 and i+2 are in flight; one barrier per step.

constexpr int kKeysPerWave = 32 * kKvHalves;
#ifndef SXA_KV_STEPS_PER_SYNC
#define SXA_KV_STEPS_PER_SYNC 2
#endif
constexpr int kStepsPerSync = SXA_KV_STEPS_PER_SYNC;  // query steps between workgroup barriers
constexpr int kStageBufs = 2 * kStepsPerSync;          // LDS stages: one group computed, one in flight
constexpr int kKeysPerWG = kKeysPerWave * kKvWaves;
constexpr int kStepRows = 32;
constexpr int kListCap = 2 * 64 * kKvWaves;  // step indices held in LDS at once
static_assert(kListCap % (64 * kKvWaves) == 0, "a list batch splits evenly over the threads");

// Stream-K list units: a tile with hits occupies kSetupUnits + hits consecutive units
// of the per-head list (the first ones stand for its setup, step list and write-back,
// so that a share that starts many short tiles gets fewer steps); a tile without
// hits, none.  Measured, a segment's fixed work takes about as long as 7 to 8 steps;
// weights 6, 7 and 8 were slower than 10 (more tiles cut), and 9 to 13 time the same.
#ifndef SXA_KV_SETUP_UNITS
#define SXA_KV_SETUP_UNITS 10
#endif
constexpr int kSetupUnits = SXA_KV_SETUP_UNITS;

struct DkdvSched {
  int32_t n_ctx_tiles, n_tiles;
  int32_t n_shares;        // stream-K workgroups; 0: one workgroup per (tile, kv head)
  const int32_t* prefix;   // [n_tiles + 1]: first list unit of each tile (per kv head)
  const int4* tinfo;       // [n_tiles]: key-coordinate range (x, y), hit steps (z) and first hit step (w)
  const int32_t* coord;    // [n_loc]: global key coordinate of each local context row
  const int32_t* share_tile;  // [n_shares]: tile holding each share's first list unit
  int32_t* hits;           // [n_tiles][hit_stride]: the hit steps of each tile, in order
                           // (nullptr when the lists would exceed kMaxListEntries: then scanned)
  int4* hits_iv;           // [n_tiles][hit_stride]: beside each listed step, the key intervals
                           // of its two blocks (as the step loop reads them from step_iv)
  int64_t hit_stride;      // query steps of a kv head (the most hits a tile can have)
  float* slots;            // [2 n_shares][kKeysPerWG][2][D]: partial dK, dV
};

// Query-step geometry of one kv head's grp query heads.
struct StepGeo {
  int gs;   // heads per token inside a step: min(grp, 32)
  int ts;   // tokens per step
  int hcs;  // steps per token (head chunks): 1 when grp <= 32
  int n_steps;
  __device__ StepGeo(int grp, int n_q) {
    gs = min(grp, kStepRows);
    ts = kStepRows / gs;
    hcs = (grp + kStepRows - 1) / kStepRows;
    n_steps = (n_q + ts - 1) / ts * hcs;
  }
  // with hcs = 1 (groups of up to 32 heads) a step is ts whole tokens; with hcs > 1,
  // ts = 1 and a token takes hcs steps: no division in the common case
  __device__ int tok0(int st) const { return hcs == 1 ? st * ts : st / hcs; }
  __device__ int h0(int st) const { return hcs == 1 ? 0 : (st % hcs) * kStepRows; }
  __device__ int ntok(int st, int n_q) const { return min(ts, n_q - tok0(st)); }
  // valid rows of a step (a prefix of its 32 rows)
  __device__ int rows(int st, int n_q, int grp) const {
    return hcs == 1 ? ntok(st, n_q) * gs : min(kStepRows, grp - h0(st));
  }
};

__device__ __forceinline__ int ld_uniform(const int32_t* ptr, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)(ptr))[i];
}

// global key coordinate of local context row `krc` (own-block tiles: the row itself)
__device__ __forceinline__ int key_coord(const BwdParams& p, bool self_tile, int64_t krc) {
  if (self_tile) return static_cast<int>(krc);
  int64_t off = 0;
  for (int c = 0; c < p.n_chunk; ++c) {
    const int len = p.chunk_len[c];
    if (krc < off + len) return p.chunk_gstart[c] + static_cast<int>(krc - off);
    off += len;
  }
  return 0;
}

__device__ __forceinline__ bool step_hit(const BwdParams& p, const StepGeo& sg, int st, int n_q,
                                         bool self_tile, int kmin, int kmax) {
  if (st >= sg.n_steps) return false;
  const int t0 = sg.tok0(st);
  const int b0 = t0 / kBlock, b1 = (t0 + sg.ntok(st, n_q) - 1) / kBlock;
  bool hit = false;
  for (int b = b0; b <= b1; ++b) {
    const int lo = self_tile ? kBlock * b : p.sample_start[b];
    const int hi = self_tile ? kBlock * b + kBlock : p.anchor[b];
    hit |= (lo <= kmax) && (hi > kmin);
  }
  return hit;
}

// Count pass: one workgroup (256 threads, one per key row) per tile.
__global__ __launch_bounds__(256) void dkdv_count_kernel(BwdParams p, DkdvSched sc, int32_t* prefix,
                                                         int4* tinfo, int32_t* coord) {
  __shared__ int red[2][4];
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid / 64;
  const bool self_tile = t >= sc.n_ctx_tiles;
  const int n_q = p.n_blk * kBlock;
  const StepGeo sg(p.hq / p.hkv, n_q);
  const int64_t key_rows = self_tile ? n_q : p.n_loc;
  const int64_t kr = static_cast<int64_t>(self_tile ? t - sc.n_ctx_tiles : t) * kKeysPerWG + tid;
  const bool valid = kr < key_rows;
  const int c = valid ? key_coord(p, self_tile, kr) : 0;
  if (valid && !self_tile) coord[kr] = c;
  int kmin = valid ? c : 0x7fffffff, kmax = valid ? c : -0x7fffffff;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, __shfl_xor(kmin, off, 64));
    kmax = max(kmax, __shfl_xor(kmax, off, 64));
  }
  if (tid % 64 == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
  kmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
  // hit steps in increasing order: batch by batch, each hit at (hits before the batch)
  // + (hits of lower waves) + (hits of lower lanes)
  int32_t* list = sc.hits != nullptr ? sc.hits + static_cast<int64_t>(t) * sc.hit_stride : nullptr;
  int4* list_iv = sc.hits != nullptr ? sc.hits_iv + static_cast<int64_t>(t) * sc.hit_stride : nullptr;
  int n = 0, first = sg.n_steps;
  for (int base = 0; base < sg.n_steps; base += 256) {
    const bool hit = step_hit(p, sg, base + tid, n_q, self_tile, kmin, kmax);
    const uint64_t m = __ballot(hit);
    __syncthreads();  // the previous batch's reads of red are done
    if (tid % 64 == 0) red[0][wave] = __popcll(m);
    __syncthreads();
    int pre = 0, cnt = 0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      pre += w2 < wave ? red[0][w2] : 0;
      cnt += red[0][w2];
    }
    if (hit) {
      const int pos = n + pre + __popcll(m & ((uint64_t{1} << (tid % 64)) - 1));
      if (list != nullptr) {
        const int st = base + tid;
        const int tk = sg.tok0(st);
        const int b0 = tk / kBlock, b1 = (tk + sg.ntok(st, n_q) - 1) / kBlock;
        list[pos] = st;
        list_iv[pos] = self_tile ? int4{kBlock * b0, kBlock * b0 + kBlock, kBlock * b1, kBlock * b1 + kBlock}
                                 : int4{p.sample_start[b0], p.anchor[b0], p.sample_start[b1], p.anchor[b1]};
      }
      if (pos == 0) red[1][0] = base + tid;  // the first hit (read after the loop)
    }
    n += cnt;
  }
  __syncthreads();
  if (n > 0) first = red[1][0];
  if (tid == 0) {
    prefix[t + 1] = n > 0 ? n + kSetupUnits : 0;
    tinfo[t] = int4{kmin, kmax, n, first};
    if (t == 0) prefix[0] = 0;
  }
}

// In-place inclusive scan of prefix[1 .. n] (one workgroup of 1024 threads), then the
// tile holding each stream-K share's first list unit (the largest tile t with
// prefix[t] <= the unit's offset in its kv head's list), so that a share starts
// without a search of its own.
__global__ __launch_bounds__(1024) void dkdv_scan_kernel(int32_t* prefix, int n, int32_t* share_tile, int n_shares,
                                                         int hkv) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = 1 + tid * per, e = min(n + 1, a + per);
  int s = 0;
  for (int i = a; i < e; ++i) s += prefix[i];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int i = a; i < e; ++i) {
    run += prefix[i];
    prefix[i] = run;
  }
  __syncthreads();  // the scanned prefix is visible to the whole workgroup
  const int64_t W = prefix[n], tot = W * hkv;
  for (int j = tid; j < n_shares && W > 0; j += 1024) {
    const int r = static_cast<int>((static_cast<int64_t>(j) * tot / n_shares) % W);
    int lo = 0, hi = n;  // prefix[lo] <= r < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (prefix[mid] <= r) lo = mid;
      else hi = mid;
    }
    share_tile[j] = lo;
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kKvWaves, 64 * kKvWaves))) void dkdv_bf16_kernel(
    BwdParams p, DkdvSched sc) {
  constexpr int H = kKvHalves;
  constexpr int kT = 64 * kKvWaves;
  constexpr int kWaves = kKvWaves;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int NI = 2 * kStepRows * CPR / kT;  // 16-byte copies per lane and step (Q, dO)
  static_assert(NI >= 1 && NI * kT == 2 * kStepRows * CPR, "stage copy must split evenly over lanes");
  constexpr int SE = 2 * kStepRows * D;  // elements of one stage: Q rows, then dO rows
  constexpr int kVCopies = kKeysPerWG * CPR / kT;  // 16-byte V tile copies per lane
  __shared__ __attribute__((aligned(256))) uint16_t vtile[kKeysPerWG * D];
  __shared__ __attribute__((aligned(256))) uint16_t stg[kStageBufs][SE];
  __shared__ __attribute__((aligned(16))) float smeta[kStageBufs][2 * kStepRows];  // lse2 rows, delta rows
  __shared__ int step_list[kListCap];
  __shared__ int4 step_iv[kListCap];  // key intervals of the listed step's two blocks
  __shared__ int kco[kKeysPerWG];     // stream-K context tiles: key coordinate of each row
  __shared__ int wave_cnt[kWaves];
  __shared__ int red[2][kWaves];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  const int grp = p.hq / p.hkv;
  const int n_q = p.n_blk * kBlock;
  const StepGeo sg(grp, n_q);

  // this workgroup's share of the (kv head, tile, hit step) list
  const bool streamk = sc.n_shares > 0;
  int share = blockIdx.x;
  int64_t W = 0, pos = 0, end = 1;
  if (streamk) {
    if (sc.n_shares % 8 == 0) share = (blockIdx.x % 8) * (sc.n_shares / 8) + blockIdx.x / 8;  // XCD-local ranges
    W = ld_uniform(sc.prefix, sc.n_tiles);
    const int64_t tot = W * p.hkv;
    pos = share * tot / sc.n_shares;
    end = (share + 1) * tot / sc.n_shares;
  }
  // element row (token * hq + head) of step row `row` relative to the step's start
  auto row_elem = [&](int row, int g) {
    const int r = min(row, (sg.hcs == 1 ? sg.ts * sg.gs : kStepRows) - 1);
    return (r / sg.gs) * p.hq + g * grp + r % sg.gs;
  };

  bool first_seg = true;  // no segment with steps yet in this share
  // (head, tile) holding list unit `pos`, the tile from the scan pass; later segments
  // are the following tiles, so the walk below only steps forward
  int g = 0, t = 0;
  if (streamk && pos < end) {
    g = static_cast<int>(pos / W);
    t = ld_uniform(sc.share_tile, share);
  }
  while (pos < end) {
    int s0, s1, hits = 0;
    int kmin, kmax;
    int scan0 = 0;  // no step before this one hits the tile
    if (streamk) {
      int r = static_cast<int>(pos - static_cast<int64_t>(g) * W);
      if (r >= W) {  // next kv head
        ++g;
        r -= static_cast<int>(W);
        t = 0;
      }
      while (ld_uniform(sc.prefix, t + 1) <= r) ++t;  // skip tiles that end at or before r
      const int u0 = ld_uniform(sc.prefix, t) + kSetupUnits, u1 = ld_uniform(sc.prefix, t + 1);
      const int ue = static_cast<int>(min<int64_t>(u1, r + (end - pos)));  // end of this share in the tile
      pos += ue - r;
      if (max(r, u0) >= ue) continue;  // only the tile's setup units fall in this share
      const int32_t* ti = reinterpret_cast<const int32_t*>(sc.tinfo) + 4 * static_cast<int64_t>(t);
      kmin = ld_uniform(ti, 0);  // scalar loads: no wait for this wave's stores in flight
      kmax = ld_uniform(ti, 1);
      hits = ld_uniform(ti, 2);
      scan0 = ld_uniform(ti, 3);
      s0 = max(r, u0) - u0;
      s1 = ue - u0;
    } else {
      g = blockIdx.x % p.hkv;
      t = blockIdx.x / p.hkv;
      s0 = 0;
      s1 = 0x7fffffff;
      pos = end;
    }
    const bool self_tile = t >= sc.n_ctx_tiles;
    const int64_t key_rows = self_tile ? n_q : p.n_loc;
    const int64_t krow0 = static_cast<int64_t>(self_tile ? t - sc.n_ctx_tiles : t) * kKeysPerWG;
    // Per-lane constants are derived anew in every segment from an opaque copy of the
    // lane index: held across segments they were spilled, and their reloads waited for
    // the previous segment's stores.
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, wave = __builtin_amdgcn_readfirstlane(tid_o / 64), lane = tid_o % 64;
    const int h2 = lane / 32, l32 = lane % 32;

    // this lane's keys (columns of the two S tiles): local rows and key coordinates
    int krow[H], kcoord[H];
    bool kvalid[H];
    int64_t krc[H];
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      krow[hh] = kKeysPerWave * wave + 32 * hh + l32;
      kvalid[hh] = krow0 + krow[hh] < key_rows;
      krc[hh] = kvalid[hh] ? krow0 + krow[hh] : key_rows - 1;
    }
    // The previous segment's pipeline ended with a barrier after its last read of
    // vtile, the list and the stages; this one only orders `red` (tile mode) and lets
    // the previous write-back stay in flight while this segment's copies start.
    lds_barrier();
    // Key coordinates: stream-K context tiles copy the count pass's coordinates of the
    // tile's rows into LDS (each lane reads its own after the pipeline's first
    // barrier, so no register waits on a load across segments); own-block tiles use
    // the row itself; without a workspace they are computed here.
    const bool kco_lds = streamk && !self_tile;
    const int last_row = static_cast<int>(min<int64_t>(kKeysPerWG, key_rows - krow0)) - 1;
#pragma unroll
    for (int hh = 0; hh < H; ++hh)
      kcoord[hh] = self_tile ? static_cast<int>(krc[hh]) : (streamk ? 0 : key_coord(p, false, krc[hh]));
    if (kco_lds && wave < kKeysPerWG / 64)
      dma4_s(sc.coord + krow0, 4u * static_cast<uint32_t>(min(wave * 64 + lane, last_row)), lds_addr(&kco[wave * 64]));
    // Stream-K: the segment's first batch of hit steps [s0, s0 + cnt0) and their key
    // intervals, copied from the count pass's lists straight into LDS (lanes past the
    // batch repeat its last entry into unused places); later batches, if any, are
    // collected by the scan below.  The tile's copies and the K loads follow, and the
    // segment waits only for the lists before it issues its first step copies: the
    // tile's loads stay in flight until the pipeline's first wait.
    int cnt0 = 0;
    if (streamk && sc.hits != nullptr) {
      cnt0 = min(kListCap, s1 - s0);
      const int64_t l0 = static_cast<int64_t>(t) * sc.hit_stride + s0;
#pragma unroll
      for (int k = 0; k < kListCap / kT; ++k) {
        const int i0 = k * kT + wave * 64;  // the wave's first entry (wave-uniform)
        if (i0 < cnt0) {
          const uint32_t i = static_cast<uint32_t>(min(i0 + lane, cnt0 - 1));
          dma4_s(sc.hits + l0, 4 * i, lds_addr(&step_list[i0]));
          dma16_s(sc.hits_iv + l0, 16 * i, lds_addr(&step_iv[i0]));
        }
      }
    }
    {  // V rows of the tile -> LDS (direct copies into the swizzled layout; rows past
       // the key rows repeat the last one)
      const uint16_t* V = (self_tile ? p.v_self : p.v) + (krow0 * p.hkv + g) * D;
#pragma unroll
      for (int j = 0; j < kVCopies; ++j) {
        const int inst = wave * kVCopies + j;
        const int c = inst * 64 + lane, row = c / CPR;
        const int logical = (c % CPR) ^ LdsTile<D>::swz(row);
        const uint32_t off = 2u * (static_cast<uint32_t>(min(row, last_row)) * static_cast<uint32_t>(p.hkv * D) +
                                   8u * static_cast<uint32_t>(logical));
        dma16_s(V, off, lds_addr(vtile + inst * 512));
      }
    }
    if (!streamk) {
      kmin = 0x7fffffff;
      kmax = -0x7fffffff;
#pragma unroll
      for (int hh = 0; hh < H; ++hh) {
        kmin = min(kmin, kvalid[hh] ? kcoord[hh] : 0x7fffffff);
        kmax = max(kmax, kvalid[hh] ? kcoord[hh] : -0x7fffffff);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        kmin = min(kmin, __shfl_xor(kmin, off, 64));
        kmax = max(kmax, __shfl_xor(kmax, off, 64));
      }
      if (lane == 0) {
        red[0][wave] = kmin;
        red[1][wave] = kmax;
      }
      lds_barrier();
      kmin = red[0][0];
      kmax = red[1][0];
#pragma unroll
      for (int w2 = 1; w2 < kWaves; ++w2) {
        kmin = min(kmin, red[0][w2]);
        kmax = max(kmax, red[1][w2]);
      }
    }

    // K of this wave's keys -> registers
    bf16x8 kf[H][KS];
    {
      const uint16_t* K = self_tile ? p.k_self : p.k;
#pragma unroll
      for (int hh = 0; hh < H; ++hh)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[hh][ks] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(K + (krc[hh] * p.hkv + g) * D + 16 * ks + 8 * h2));
    }
    // The list copies are done once at most the kVCopies + H KS loads issued after them
    // are in flight (vector loads complete in issue order); the compiler barrier keeps
    // those K loads above the wait.
    asm volatile("" ::: "memory");
    wait_vmcnt<kVCopies + H * KS>();
    f32x16 dkacc[H][DT], dvacc[H][DT];
#pragma unroll
    for (int hh = 0; hh < H; ++hh)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dkacc[hh][dt][i] = dvacc[hh][dt][i] = 0.f;

    // Copy sources: byte offset of each lane from the step's first element (rows
    // past the step's used rows repeat its last row; all are masked)
    int src_off[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int cc = ((wave * NI + j) * 64 + lane) % (kStepRows * CPR), row = cc / CPR;
      const int logical = (cc % CPR) ^ LdsTile<D>::swz(row);
      src_off[j] = 2 * (row_elem(row, g) * D + 8 * logical);
    }
    // wave 0, lanes 0..31: lse2 plane of row l32; lanes 32..63: delta plane
    const int meta_off = 4 * row_elem(l32, g);
    const int plane_off = h2 == 0 ? 4 * n_q * p.hq : 0;

    // LDS byte offsets (see LdsTile): Q / dO row l32, V rows krow, transposed reads
    int f_q = LdsTile<D>::frag_off(l32, h2);
    int f_v = LdsTile<D>::frag_off(krow[0], h2);  // second half: + 32 rows
    int t_a = LdsTile<D>::tr_off(4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
    int t_b = LdsTile<D>::tr_off(8 + 4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
    int rel = 4 * h2;  // step row of accumulator row 4 j + i: 8 j + rel + i

    int scan = scan0;  // next step to examine
    int ord = 0;       // hits of this tile before `scan`
    bool listed = cnt0 > 0;  // the first batch is in LDS already
    while (scan < sg.n_steps && ord < s1) {
      // ---- collect the step indices of hits ord in [s0, s1), up to the list capacity
      int cnt = 0;
      const bool from_list = listed;
      if (listed) {
        lds_barrier();  // the listed batch is visible to every wave
        cnt = cnt0;
        ord = s0 + cnt0;                                                     // hits before `scan`
        scan = __builtin_amdgcn_readfirstlane(step_list[cnt0 - 1]) + 1;  // past the last listed hit
        listed = false;
      }
      while (!from_list && scan < sg.n_steps && ord < s1 && cnt <= kListCap - kT) {
        const int st = scan + tid;
        const bool hit = step_hit(p, sg, st, n_q, self_tile, kmin, kmax);
        const uint64_t m = __ballot(hit);
        if (lane == 0) wave_cnt[wave] = __popcll(m);
        lds_barrier();
        int pre = 0, tot = 0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
          const int cw = wave_cnt[w2];
          pre += w2 < wave ? cw : 0;
          tot += cw;
        }
        const int o = ord + pre + __popcll(m & ((uint64_t{1} << lane) - 1));
        const int first = max(ord, s0);
        if (hit && o >= s0 && o < s1) {
          const int tk = sg.tok0(st);
          const int b0 = tk / kBlock, b1 = (tk + sg.ntok(st, n_q) - 1) / kBlock;
          step_list[cnt + o - first] = st;
          step_iv[cnt + o - first] =
              self_tile ? int4{kBlock * b0, kBlock * b0 + kBlock, kBlock * b1, kBlock * b1 + kBlock}
                        : int4{p.sample_start[b0], p.anchor[b0], p.sample_start[b1], p.anchor[b1]};
        }
        cnt += max(0, min(ord + tot, s1) - first);
        ord += tot;
        scan += kT;
        lds_barrier();
      }

      // ---- pipeline over the listed steps in groups of kStepsPerSync: iteration j
      // waits for group j (every load of this wave, the tile's included), copies group
      // j + 1 into the stages group j - 1 used, then computes group j.
      const int ngrp = (cnt + kStepsPerSync - 1) / kStepsPerSync;
      for (int jg = -1; jg < ngrp; ++jg) {
        if (jg >= 0) {
          wait_vmcnt<0>();    // this wave's copies of group jg landed
          barrier_nofence();  // every wave's; group jg - 1's stages are no longer read
          if (jg == 0 && kco_lds) {  // the tile's copies (coordinates included) have landed
#pragma unroll
            for (int hh = 0; hh < H; ++hh) kcoord[hh] = kco[krow[hh]];
          }
        }
#pragma unroll
        for (int q = 0; q < kStepsPerSync; ++q) {
          const int si = (jg + 1) * kStepsPerSync + q;
          if (jg + 1 >= ngrp || si >= cnt) break;
          const int nst = __builtin_amdgcn_readfirstlane(step_list[si]);
          const int sb2 = si % kStageBufs;
          const int64_t e0 = static_cast<int64_t>(sg.tok0(nst)) * p.hq + sg.h0(nst);  // first element row
          // clamp to the arrays (rows past the end are masked)
          const int lim_q = static_cast<int>(min<int64_t>(0x7fffffff, 2 * ((static_cast<int64_t>(n_q) * p.hq - e0) * D - 8)));
          const int lim_m = static_cast<int>(4 * (static_cast<int64_t>(n_q) * p.hq - e0 - 1));
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const bool is_do = (wave * NI + j) * 64 >= kStepRows * CPR;  // wave-uniform
            dma16_s((is_do ? p.dout : p.q) + e0 * D, static_cast<uint32_t>(min(src_off[j], lim_q)),
                    lds_addr(stg[sb2] + (wave * NI + j) * 512));
          }
          if (wave == 0)
            dma4_s(p.delta + e0, static_cast<uint32_t>(min(meta_off, lim_m) + plane_off), lds_addr(&smeta[sb2][0]));
        }
        if (jg < 0) continue;

#pragma unroll 1
        for (int q = 0; q < kStepsPerSync; ++q) {
        const int i = jg * kStepsPerSync + q;
        if (i >= cnt) break;
        // Per-lane constants are redefined opaquely every step so that the compiler
        // recomputes the few values derived from them instead of holding dozens.
        asm volatile("" : "+v"(f_q), "+v"(f_v), "+v"(t_a), "+v"(t_b), "+v"(rel));
        const int sb = i % kStageBufs;
        const int st = __builtin_amdgcn_readfirstlane(step_list[i]);
        const int tk = sg.tok0(st);
        const int rmax = sg.rows(st, n_q, grp);
        const int b0 = tk / kBlock;
        const int split = (kBlock * (b0 + 1) - tk) * sg.gs;  // rows < split are in block b0
        const int4 iv = step_iv[i];
        const int lo0 = __builtin_amdgcn_readfirstlane(iv.x), hi0 = __builtin_amdgcn_readfirstlane(iv.y);
        const int lo1 = __builtin_amdgcn_readfirstlane(iv.z), hi1 = __builtin_amdgcn_readfirstlane(iv.w);
        bool ok0[H], ok1[H], any = false, all = true;
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
          ok0[hh] = kvalid[hh] && kcoord[hh] >= lo0 && kcoord[hh] < hi0;
          ok1[hh] = kvalid[hh] && kcoord[hh] >= lo1 && kcoord[hh] < hi1;
          any |= ok0[hh] || ok1[hh];
          all &= ok0[hh] && ok1[hh];
        }
        if (!__any(any)) continue;
        const bool all_ok = rmax == kStepRows && __all(all);
        // Per-step LDS base addresses: stage bases are 16 KB aligned, so the k-step
        // parts of the swizzled offsets (XOR constants) apply to base + offset; the
        // dO rows (+ 32 D * 2 bytes) and later k-steps of the transposed reads are
        // immediate offsets.
        constexpr uint32_t kDoOff = kStepRows * D * 2;
        const uint32_t stage = lds_addr(stg[sb]);
        const uint32_t qb = stage + f_q, ta = stage + t_a, tb = stage + t_b;
        const uint32_t vbase = lds_addr(vtile) + f_v;
        f32x16 sacc[H], pacc[H];
#pragma unroll
        for (int hh = 0; hh < H; ++hh)
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) sacc[hh][i2] = pacc[hh][i2] = 0.f;
        // operands are read one k-step ahead; the scheduling barriers keep the compiler
        // from hoisting every k-step's reads (register pressure)
        bf16x8 qa = lds_frag(qb), da = lds_frag(qb + kDoOff);
        bf16x8 vb[H];
#pragma unroll
        for (int hh = 0; hh < H; ++hh) vb[hh] = lds_frag(vbase + hh * 64 * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 cq = qa, cd = da;
          bf16x8 cv[H];
#pragma unroll
          for (int hh = 0; hh < H; ++hh) cv[hh] = vb[hh];
          if (ks + 1 < KS) {
            const uint32_t o = qb ^ (32 * (ks + 1)), ov = vbase ^ (32 * (ks + 1));
            qa = lds_frag(o);
            da = lds_frag(o + kDoOff);
#pragma unroll
            for (int hh = 0; hh < H; ++hh) vb[hh] = lds_frag(ov + hh * 64 * D);
          }
#pragma unroll
          for (int hh = 0; hh < H; ++hh) {
            sacc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cq, kf[hh][ks], sacc[hh], 0, 0, 0);
            pacc[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cd, cv[hh], pacc[hh], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // exponent S scale log2 e - lse2, in place
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&smeta[sb][8 * j + 4 * h2]);  // rows 8 j + 4 h2 + 0..3
#pragma unroll
          for (int hh = 0; hh < H; ++hh)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) sacc[hh][4 * j + i2] = fmaf(sacc[hh][4 * j + i2], p.scale_log2, -l4[i2]);
        }
        if (!all_ok) {  // keys outside a row's interval (and padding rows) get exp2(-inf) = 0
#pragma unroll
          for (int hh = 0; hh < H; ++hh)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 8 * (r / 4) + r % 4;  // row 8 j + rel + i
              const bool ok = (rel < split - c ? ok0[hh] : ok1[hh]) && rel < rmax - c;
              sacc[hh][r] = ok ? sacc[hh][r] : -INFINITY;
            }
        }
        // P = exp2(.) and dS = P (dP - delta) as bf16 pairs.  Accumulator rows 8 j +
        // rel + (0..3) of j = 0, 1 feed the dV, dK products' first k-half (kq = 0), those
        // of j = 2, 3 the second; the second half's exponents and products are formed
        // between the first half's MFMAs (four quarters of two rows over its DT k-steps).
        u32x4 pw[H][2], sw[H][2];
        auto p_ds = [&](int j, int half, const f32x4& d4) {
#pragma unroll
          for (int hh = 0; hh < H; ++hh) {
            const int r = 4 * j + 2 * half;
            const float p0 = __builtin_amdgcn_exp2f(sacc[hh][r]), p1 = __builtin_amdgcn_exp2f(sacc[hh][r + 1]);
            const float s0 = p0 * (pacc[hh][r] - d4[2 * half]), s1 = p1 * (pacc[hh][r + 1] - d4[2 * half + 1]);
            pw[hh][j / 2][2 * (j % 2) + half] = pack_bf16x2(p0, p1);
            sw[hh][j / 2][2 * (j % 2) + half] = pack_bf16x2(s0, s1);
          }
        };
        f32x4 d4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d4[j] = *reinterpret_cast<const f32x4*>(&smeta[sb][kStepRows + 8 * j + 4 * h2]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          p_ds(j, 0, d4[j]);
          p_ds(j, 1, d4[j]);
        }
        bf16x8 dta = lds_frag_t(ta + kDoOff, tb + kDoOff), qta = lds_frag_t(ta, tb);
#pragma unroll
        for (int kd = 0; kd < 2 * DT; ++kd) {
          const int kq = kd / DT, dt = kd % DT;
          const bf16x8 cdt = dta, cqt = qta;
          if (kd + 1 < 2 * DT) {
            const int kq1 = (kd + 1) / DT, dt1 = (kd + 1) % DT;
            const uint32_t oa = (ta ^ (64 * dt1)) + kq1 * 32 * D, ob = (tb ^ (64 * dt1)) + kq1 * 32 * D;
            dta = lds_frag_t(oa + kDoOff, ob + kDoOff);
            qta = lds_frag_t(oa, ob);
          }
#pragma unroll
          for (int hh = 0; hh < H; ++hh) {
            dvacc[hh][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cdt, __builtin_bit_cast(bf16x8, pw[hh][kq]),
                                                                    dvacc[hh][dt], 0, 0, 0);
            dkacc[hh][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cqt, __builtin_bit_cast(bf16x8, sw[hh][kq]),
                                                                    dkacc[hh][dt], 0, 0, 0);
          }
          // the second k-half's four quarters, spread over the first half's DT k-steps
#pragma unroll
          for (int qq = 4 * kd / DT; qq < 4 * (kd + 1) / DT && kd < DT; ++qq) p_ds(2 + qq / 2, qq % 2, d4[2 + qq / 2]);
          __builtin_amdgcn_sched_barrier(0);
        }
        }  // steps of the group
      }
      __syncthreads();  // all waves are done with the list and the stages
    }

    // ---- epilogue: whole tile -> dK, dV; partial -> this share's slot
    const bool whole = !streamk || (s0 == 0 && s1 == hits);
    float* slot = nullptr;
    if (!whole)
      slot = sc.slots + (2 * static_cast<int64_t>(share) + (first_seg ? 0 : 1)) *
                            (static_cast<int64_t>(kKeysPerWG) * 2 * D);
    first_seg = false;
#pragma unroll
    for (int hh = 0; hh < H; ++hh) {
      if (!kvalid[hh]) continue;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int dcol = 32 * dt + 8 * jj + 4 * h2;
          const f32x4 kv4 = f32x4{dkacc[hh][dt][4 * jj], dkacc[hh][dt][4 * jj + 1], dkacc[hh][dt][4 * jj + 2],
                                  dkacc[hh][dt][4 * jj + 3]};
          const f32x4 vv4 = f32x4{dvacc[hh][dt][4 * jj], dvacc[hh][dt][4 * jj + 1], dvacc[hh][dt][4 * jj + 2],
                                  dvacc[hh][dt][4 * jj + 3]};
          if (whole) {
            const int64_t o = ((krow0 + krow[hh]) * p.hkv + g) * D + dcol;
            store_grad4(self_tile ? p.dk_self : p.dk, o, kv4 * p.scale, p.grad_bf16);
            store_grad4(self_tile ? p.dv_self : p.dv, o, vv4, p.grad_bf16);
          } else {
            *reinterpret_cast<f32x4*>(slot + (krow[hh] * 2 + 0) * D + dcol) = kv4;
            *reinterpret_cast<f32x4*>(slot + (krow[hh] * 2 + 1) * D + dcol) = vv4;
          }
        }
    }
  }
}

// Stream-K fix-up: kRedParts workgroups per (tile, kv head), each over a contiguous
// part of the tile's dK, dV rows.  Tiles no step hits get dK = dV = 0; tiles split
// over several shares get the sum of those shares' slots.
constexpr int kRedParts = 16;

template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(BwdParams p, DkdvSched sc) {
  constexpr int V4 = kKeysPerWG * 2 * D / 4;  // float4 of one tile's dK, dV
  constexpr int PER = V4 / kRedParts;
  static_assert(PER % 256 == 0, "parts must split evenly over the threads");
  const int part = blockIdx.x % kRedParts;
  const int g = (blockIdx.x / kRedParts) % p.hkv;
  const int t = blockIdx.x / kRedParts / p.hkv;
  const bool self_tile = t >= sc.n_ctx_tiles;
  const int64_t n_q = static_cast<int64_t>(p.n_blk) * kBlock;
  const int64_t key_rows = self_tile ? n_q : p.n_loc;
  const int64_t krow0 = static_cast<int64_t>(self_tile ? t - sc.n_ctx_tiles : t) * kKeysPerWG;
  void* dK = self_tile ? p.dk_self : p.dk;
  void* dV = self_tile ? p.dv_self : p.dv;
  const int64_t W = ld_uniform(sc.prefix, sc.n_tiles);
  const int t0 = ld_uniform(sc.prefix, t);
  const int hits = sc.tinfo[t].z;
  int64_t j0 = 0, j1 = 0;
  bool j0_later = false;
  const int64_t tot = W * p.hkv, ns = sc.n_shares;
  if (hits > 0) {
    // the tile's steps are list units [G0, G1) of the flattened (head, tile) list
    const int64_t G0 = static_cast<int64_t>(g) * W + t0 + kSetupUnits, G1 = G0 + hits;
    // share j covers [floor(j tot / ns), floor((j + 1) tot / ns)); share holding x:
    j0 = ((G0 + 1) * ns - 1) / tot;
    j1 = (G1 * ns - 1) / tot;
    if (j0 == j1) return;  // one share covered the whole tile and wrote it
    // share j0 had steps of an earlier tile when it starts before this tile's units
    j0_later = j0 * tot / ns < G0 - kSetupUnits;
  }
  const int64_t slot_elems = static_cast<int64_t>(kKeysPerWG) * 2 * D;
#pragma unroll 2
  for (int i = part * PER + threadIdx.x; i < (part + 1) * PER; i += 256) {
    const int e = 4 * i;
    const int krow = e / (2 * D), which = (e / D) % 2, dcol = e % D;
    const int64_t kr = krow0 + krow;
    if (kr >= key_rows) continue;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (hits > 0) {
      acc = *reinterpret_cast<const f32x4*>(sc.slots + (2 * j0 + (j0_later ? 1 : 0)) * slot_elems + e);
      for (int64_t j = j0 + 1; j <= j1; ++j)
        if ((j + 1) * tot / ns > j * tot / ns)  // empty shares (list shorter than the grid) wrote nothing
          acc += *reinterpret_cast<const f32x4*>(sc.slots + 2 * j * slot_elems + e);
    }
    store_grad4(which == 0 ? dK : dV, (kr * p.hkv + g) * D + dcol, which == 0 ? acc * p.scale : acc, p.grad_bf16);
  }
}

// Hit lists (a step index and its blocks' key intervals, 20 bytes per entry) are kept
// up to this many (tile, step) entries (320 MiB); larger calls scan.
constexpr int64_t kMaxListEntries = int64_t{1} << 24;

struct WsLayout {
  int64_t n_tiles, n_shares, hit_stride, prefix_off, tinfo_off, coord_off, share_off, hits_off, hits_iv_off,
      order_off, slots_off, bytes;
  bool lists;
};

WsLayout ws_layout(int64_t n_blk, int64_t n_loc, int64_t d, int64_t grp) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  WsLayout L;
  L.n_tiles = (n_loc + kKeysPerWG - 1) / kKeysPerWG + (n_blk * kBlock + kKeysPerWG - 1) / kKeysPerWG;
  L.n_shares = n_compute_units();
  const int64_t groups = (n_blk * kBlock * grp + kRowsPerGroup - 1) / kRowsPerGroup;
  {  // query steps of one kv head, as StepGeo counts them
    const int64_t gs = grp < kStepRows ? grp : kStepRows, ts = kStepRows / gs;
    const int64_t hcs = (grp + kStepRows - 1) / kStepRows;
    L.hit_stride = (n_blk * kBlock + ts - 1) / ts * hcs;
  }
  L.prefix_off = 0;
  L.tinfo_off = up(4 * (L.n_tiles + 1));
  L.coord_off = L.tinfo_off + up(16 * L.n_tiles);
  L.share_off = L.coord_off + up(4 * n_loc);
  L.hits_off = L.share_off + up(4 * L.n_shares);
  L.lists = L.n_tiles * L.hit_stride <= kMaxListEntries;
  L.hits_iv_off = L.hits_off + (L.lists ? up(4 * L.n_tiles * L.hit_stride) : 0);
  L.order_off = L.hits_iv_off + (L.lists ? up(16 * L.n_tiles * L.hit_stride) : 0);
  L.slots_off = L.order_off + up(4 * (groups < kMaxOrderedGroups ? groups : int64_t{kMaxOrderedGroups}));
  L.bytes = L.slots_off + 2 * L.n_shares * static_cast<int64_t>(kKeysPerWG) * 2 * d * 4;
  return L;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (a.flags & SXA_BWD_DELTA) {
    if ((e = launch_delta(a, true, s)) != hipSuccess) return e;
  }
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.k_self = static_cast<const uint16_t*>(a.k_self);
  p.v_self = static_cast<const uint16_t*>(a.v_self);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse_in;
  p.delta = a.delta;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dk_self = a.dk_self;
  p.dv_self = a.dv_self;
  p.grad_bf16 = (a.flags & SXA_BWD_DKDV_BF16) != 0;
  p.anchor = a.anchor;
  p.sample_start = a.sample_start;
  p.chunk_gstart = a.chunk_gstart;
  p.chunk_len = a.chunk_len;
  p.n_loc = a.n_loc;
  p.n_blk = a.n_blk;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.n_chunk = a.n_chunk;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.dq_overwrite = (a.flags & SXA_BWD_DQ_OVERWRITE) != 0;
  p.rg_order = nullptr;
  p.jobs = nullptr;
  p.part_dq = nullptr;
  if (a.flags & SXA_BWD_DQ) {
    static_assert(32 * kDqWaves == kRowsPerGroup, "row groups are shared with the dispatch order");
    const int64_t groups = row_groups(a, kRowsPerGroup);
    const int64_t n_dq = groups * a.hkv;
    if (a.row_split != nullptr && groups <= kMaxOrderedGroups && groups > 0) {
      const RowSplit sp = row_split_layout(a.row_split, a);
      if ((e = launch_row_split_plan(a, sp, s)) != hipSuccess) return e;
      p.jobs = sp.jobs;
      p.part_dq = sp.part_o;
      dq_bf16_kernel<D><<<dim3(static_cast<unsigned>((groups + sp.max_extra) * a.hkv)), dim3(64 * kDqWaves), 0, s>>>(p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      constexpr int kRuns = kRowsPerGroup / (256 / (D / 4));
      dq_merge_kernel<D><<<dim3(static_cast<unsigned>(a.hkv * kRuns)), dim3(256), 0, s>>>(sp, a.dq, a.n_blk, a.hq,
                                                                                          a.hkv, p.dq_overwrite);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      p.jobs = nullptr;
    } else if (a.workspace != nullptr && groups <= kMaxOrderedGroups) {
      const WsLayout L = ws_layout(a.n_blk, a.n_loc, D, a.hq / a.hkv);
      int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) + L.order_off);
      if ((e = launch_row_group_order(a, kRowsPerGroup, order, s)) != hipSuccess) return e;
      p.rg_order = order;
    }
    if (p.part_dq == nullptr) {
      dq_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_dq)), dim3(64 * kDqWaves), 0, s>>>(p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (!(a.flags & SXA_BWD_DKDV)) return hipSuccess;
  const int64_t n_ctx_tiles = (a.n_loc + kKeysPerWG - 1) / kKeysPerWG;
  const int64_t n_q = static_cast<int64_t>(a.n_blk) * kBlock;
  const int64_t n_self_tiles = a.k_self ? (n_q + kKeysPerWG - 1) / kKeysPerWG : 0;
  const int64_t n_tiles = n_ctx_tiles + n_self_tiles;
  if (n_tiles == 0) return hipSuccess;
  DkdvSched sc;
  sc.n_ctx_tiles = static_cast<int32_t>(n_ctx_tiles);
  sc.n_tiles = static_cast<int32_t>(n_tiles);
  sc.n_shares = 0;
  sc.prefix = nullptr;
  sc.tinfo = nullptr;
  sc.coord = nullptr;
  sc.share_tile = nullptr;
  sc.hits = nullptr;
  sc.hits_iv = nullptr;
  sc.hit_stride = 0;
  sc.slots = nullptr;
  if (a.workspace != nullptr) {
    const WsLayout L = ws_layout(a.n_blk, a.n_loc, D, a.hq / a.hkv);
    char* ws = static_cast<char*>(a.workspace);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + L.prefix_off);
    int4* tinfo = reinterpret_cast<int4*>(ws + L.tinfo_off);
    int32_t* coord = reinterpret_cast<int32_t*>(ws + L.coord_off);
    sc.n_shares = static_cast<int32_t>(L.n_shares);
    sc.prefix = prefix;
    sc.tinfo = tinfo;
    sc.coord = coord;
    int32_t* share_tile = reinterpret_cast<int32_t*>(ws + L.share_off);
    sc.share_tile = share_tile;
    sc.hits = L.lists ? reinterpret_cast<int32_t*>(ws + L.hits_off) : nullptr;
    sc.hits_iv = L.lists ? reinterpret_cast<int4*>(ws + L.hits_iv_off) : nullptr;
    sc.hit_stride = L.hit_stride;
    sc.slots = reinterpret_cast<float*>(ws + L.slots_off);
    dkdv_count_kernel<<<dim3(static_cast<unsigned>(n_tiles)), dim3(256), 0, s>>>(p, sc, prefix, tinfo, coord);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dkdv_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(prefix, static_cast<int>(n_tiles), share_tile,
                                                    static_cast<int>(L.n_shares), a.hkv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dkdv_bf16_kernel<D><<<dim3(static_cast<unsigned>(L.n_shares)), dim3(64 * kKvWaves), 0, s>>>(p, sc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dkdv_reduce_kernel<D><<<dim3(static_cast<unsigned>(n_tiles * a.hkv * kRedParts)), dim3(256), 0, s>>>(p, sc);
    return hipGetLastError();
  }
  dkdv_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_tiles * a.hkv)), dim3(64 * kKvWaves), 0, s>>>(p, sc);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_bytes(int32_t n_blk, int64_t n_loc, int32_t hq, int32_t hkv, int32_t d) {
  return ws_layout(n_blk, n_loc, d, hq / hkv).bytes;
}

hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace sxa
