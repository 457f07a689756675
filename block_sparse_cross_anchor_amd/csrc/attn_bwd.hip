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
#include "lds_tile.h"

namespace sxa {
namespace {

constexpr int kTileKeys = 64;
#ifndef SXA_DQ_WAVES
#define SXA_DQ_WAVES 8
#endif
#ifndef SXA_KV_WAVES
#define SXA_KV_WAVES 8
#endif
constexpr int kDqWaves = SXA_DQ_WAVES;  // waves per dq workgroup (32 query rows each)
constexpr int kKvWaves = SXA_KV_WAVES;  // waves per dkdv workgroup (32 keys each)

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_self;
  const uint16_t* v_self;
  const uint16_t* dout;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  float* dk_self;
  float* dv_self;
  const int32_t* anchor;
  const int32_t* sample_start;
  const int32_t* chunk_gstart;
  const int32_t* chunk_len;
  int64_t n_loc;
  int32_t n_blk, hq, hkv, n_chunk;
  float scale;
  float scale_log2;  // scale * log2(e)
  int32_t dq_overwrite;
  int32_t* ws_parts;  // dK/dV split scratch: parts per (context tile, kv head), or nullptr
  float* ws_slots;    // [tile][hkv][kMaxParts][keys per tile][2][D] partial dK, dV
};

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

// ============================================================================ dq kernel

struct Tile {
  int64_t row0;
  int nrows;
  int coord0;
  int self;
};

struct Walk {
  int self_pos, self_end;
  int c;
  int64_t off;
  int gs, len, t, t_end;
};

__device__ __forceinline__ bool walk_next(Walk& w, const int32_t* __restrict__ cgs,
                                          const int32_t* __restrict__ clen, int n_chunk, int LO,
                                          int HI, Tile& out) {
  if (w.self_pos < w.self_end) {
    out.row0 = w.self_pos;
    out.nrows = min(kTileKeys, w.self_end - w.self_pos);
    out.coord0 = w.self_pos;
    out.self = 1;
    w.self_pos += kTileKeys;
    return true;
  }
  while (true) {
    if (w.t < w.t_end) {
      out.row0 = w.off + static_cast<int64_t>(w.t) * kTileKeys;
      out.nrows = min(kTileKeys, w.len - w.t * kTileKeys);
      out.coord0 = w.gs + w.t * kTileKeys;
      out.self = 0;
      ++w.t;
      return true;
    }
    if (w.c >= n_chunk) return false;
    w.off += w.len;
    ++w.c;
    if (w.c >= n_chunk) {
      w.len = 0;
      return false;
    }
    w.gs = cgs[w.c];
    w.len = clen[w.c];
    const int a = max(LO, w.gs), e = min(HI, w.gs + w.len);
    if (a < e) {
      w.t = (a - w.gs) / kTileKeys;
      w.t_end = (e - w.gs + kTileKeys - 1) / kTileKeys;
    } else {
      w.t = w.t_end = 0;
    }
  }
}

// K and V tiles staged row-major (lds_tile.h); K^T for dQ comes from the
// transposing read of the same K tile.
template <int D, int kT>
struct DqTileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int CH = kTileKeys * CPR;
  static constexpr int L = (CH + kT - 1) / kT;
  u32x4 k[L], v[L];

  __device__ __forceinline__ void load(const Tile& t, const BwdParams& p, int g, int tid) {
    const uint16_t* K = t.self ? p.k_self : p.k;
    const uint16_t* V = t.self ? p.v_self : p.v;
    const int last = t.nrows - 1;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int idx = tid + kT * i;
      if (CH % kT == 0 || idx < CH) {
        const int key = min(idx / CPR, last), j = idx % CPR;
        const int64_t off = ((t.row0 + key) * p.hkv + g) * D + 8 * j;
        k[i] = *reinterpret_cast<const u32x4*>(K + off);
        v[i] = *reinterpret_cast<const u32x4*>(V + off);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lk, uint16_t* lv, int tid) const {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int idx = tid + kT * i;
      if (CH % kT == 0 || idx < CH) {
        LdsTile<D>::store(lk, idx / CPR, idx % CPR, k[i]);
        LdsTile<D>::store(lv, idx / CPR, idx % CPR, v[i]);
      }
    }
  }
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kDqWaves, 64 * kDqWaves))) void dq_bf16_kernel(
    BwdParams p) {
  constexpr int kT = 64 * kDqWaves;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int ROWS = 32 * kDqWaves;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTileKeys * D];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  const int g = blockIdx.x % p.hkv;
  const int wg = blockIdx.x / p.hkv;
  const int grp = p.hq / p.hkv;
  const int64_t R = static_cast<int64_t>(p.n_blk) * kBlock * grp;
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
  w.self_pos = p.k_self ? kBlock * b_first : 0;
  w.self_end = p.k_self ? kBlock * (b_last + 1) : 0;
  w.c = -1;
  w.off = 0;
  w.gs = w.len = w.t = w.t_end = 0;
  Tile cur, nxt;
  bool have = walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, cur);

  // this lane's query row (column of the 32-row N tile)
  const int64_t r = wg_row0 + 32 * wave + l32;
  const bool valid = r < R;
  const int64_t rr = valid ? r : 0;
  const int64_t tok = rr / grp;
  const int hh = static_cast<int>(rr % grp);
  const int blk = static_cast<int>(tok / kBlock);
  const int64_t orow = tok * p.hq + static_cast<int64_t>(g) * grp + hh;
  if (!have) {  // no key of this call reaches these rows: nothing to add
    if (p.dq_overwrite && valid) {
      // the two lanes of a row (h2 = 0, 1) each clear half of it
#pragma unroll
      for (int d0 = h2 * (D / 2); d0 < (h2 + 1) * (D / 2); d0 += 4)
        *reinterpret_cast<f32x4*>(p.dq + orow * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int clo = valid ? p.sample_start[blk] : 0, chi = valid ? p.anchor[blk] : 0;
  const int slo = valid ? kBlock * blk : 0, shi = valid ? kBlock * blk + kBlock : 0;
  const float lse_nat = p.lse[orow];
  // rows with no key at all contribute nothing: exp2(x - inf) = 0
  const float lse2 = (valid && lse_nat != -INFINITY) ? lse_nat * kLog2e : INFINITY;
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

  DqTileRegs<D, kT> regs;
  regs.load(cur, p, g, tid);
  regs.store(lds[0][0], lds[0][1], tid);
  __syncthreads();
  int buf = 0;
  while (have) {
    const bool has_next = walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, nxt);
    if (has_next) regs.load(nxt, p, g, tid);

    const int lo = cur.self ? slo : clo, hi = cur.self ? shi : chi;
    const int a_lo = max(lo - cur.coord0, 0), a_hi = min(hi - cur.coord0, cur.nrows);
    const bool any = a_lo < a_hi;
    const bool full = (a_lo == 0) & (a_hi == kTileKeys);
    if (__any(any)) {
      const bool all_full = __all(full);
      const uint16_t* lk = lds[buf][0];
      const uint16_t* lv = lds[buf][1];
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mt][i] = pacc[mt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 kf = LdsTile<D>::frag(lk, 32 * mt + l32, 2 * ks + h2);
          const bf16x8 vf = LdsTile<D>::frag(lv, 32 * mt + l32, 2 * ks + h2);
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
          pacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[ks], pacc[mt], 0, 0, 0);
        }
      }
      bf16x8 dsf[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pr = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], p.scale_log2, -lse2));
          if (!all_full) {
            const int key = 32 * mt + 8 * (i / 4) + 4 * h2 + (i % 4);
            if (key < a_lo || key >= a_hi) pr = 0.f;
          }
          const float ds = pr * (pacc[mt][i] - dlt);
          dsf[2 * mt + i / 8][i % 8] = static_cast<__bf16>(ds);
        }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int sl = lane & 15;
          const bf16x8 kt = LdsTile<D>::frag_t(lk, tr_row_a(kq, h2, sl), tr_row_b(kq, h2, sl),
                                               32 * dt + 16 * ((lane >> 4) & 1), sl);
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[kq], dqacc[dt], 0, 0, 0);
        }
      }
    }

    if (has_next) regs.store(lds[buf ^ 1][0], lds[buf ^ 1][1], tid);
    __syncthreads();
    if (!has_next) break;
    cur = nxt;
    buf ^= 1;
  }

  if (!valid) return;
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

// ============================================================================ dkdv kernel
//
// Workgroup: 8 waves x 32 keys = 256 consecutive key rows of one kv head (local
// context rows, or own-block rows for the tiles after the context ones).  K of a
// wave's keys is held in registers (MFMA B operand of S = Q K^T); V of the
// workgroup's keys sits in LDS (B operand of dP = dO V^T).  Query rows of kv head
// g are numbered r = token * grp + (h - g*grp) and visited in steps of 32 rows;
// a step is visited when one of its blocks' key intervals meets the workgroup's
// keys (own-block tiles: when it holds one of their blocks).  When the group size
// is even a step lies inside one block, so its mask is one interval ("uniform").

constexpr int kKeysPerWG = 32 * kKvWaves;
constexpr int kStepRows = 32;
constexpr int kStepsPerPart = 112;  // query steps per workgroup above which a tile is split
constexpr int kMaxParts = 4;

struct StepMeta {
  float lse2[kStepRows];  // log2-domain lse per row (+inf: row contributes nothing)
  float dlt[kStepRows];   // delta per row
  int lo[kStepRows];      // per-row allowed key interval (non-uniform steps)
  int hi[kStepRows];
  int uni, lo0, hi0;      // uniform step: one interval for all rows
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kKvWaves, 64 * kKvWaves))) void dkdv_bf16_kernel(BwdParams p,
                                                                                      int n_ctx_tiles,
                                                                                      int n_tiles) {
  constexpr int kT = 64 * kKvWaves;
  constexpr int kWaves = kKvWaves;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  constexpr int SCH = 2 * kStepRows * CPR;  // 16-byte chunks of Q and dO rows of one step
  constexpr int SL = (SCH + kT - 1) / kT;
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kKeysPerWG * D];
  // per stage: Q and dO rows of the step, row-major (transposed operands via tr reads)
  __shared__ __attribute__((aligned(16))) uint16_t stg[2][2][kStepRows * D];
  __shared__ __attribute__((aligned(16))) StepMeta meta[2];
  __shared__ int step_list[kT];
  __shared__ int wave_cnt[kWaves];
  __shared__ int red[2][kWaves];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  // blockIdx -> (part, tile, kv head); all first parts are dispatched first
  const int per_part = n_tiles * p.hkv;
  const int part = blockIdx.x / per_part;
  const int g = (blockIdx.x % per_part) % p.hkv;
  const int tile = (blockIdx.x % per_part) / p.hkv;
  const bool self_tile = tile >= n_ctx_tiles;
  const int grp = p.hq / p.hkv;
  const int64_t n_q = static_cast<int64_t>(p.n_blk) * kBlock;
  const int64_t R = n_q * grp;
  const int64_t n_steps = (R + kStepRows - 1) / kStepRows;
  const int64_t key_rows = self_tile ? n_q : p.n_loc;
  const int64_t krow0 = static_cast<int64_t>(self_tile ? tile - n_ctx_tiles : tile) * kKeysPerWG;
  const uint16_t* K = self_tile ? p.k_self : p.k;
  const uint16_t* V = self_tile ? p.v_self : p.v;

  // this lane's key (column of the S tile): local row and key coordinate
  const int krow = 32 * wave + l32;
  const int64_t kr = krow0 + krow;
  const bool kvalid = kr < key_rows;
  const int64_t krc = kvalid ? kr : key_rows - 1;
  int kcoord = 0;  // global position (context) or own-block row (self)
  if (self_tile) {
    kcoord = static_cast<int>(krc);
  } else {
    int64_t off = 0;
    for (int c = 0; c < p.n_chunk; ++c) {
      const int len = p.chunk_len[c];
      if (krc < off + len) {
        kcoord = p.chunk_gstart[c] + static_cast<int>(krc - off);
        break;
      }
      off += len;
    }
  }
  // key-coordinate range of the workgroup
  int kmin = kvalid ? kcoord : 0x7fffffff, kmax = kvalid ? kcoord : -0x7fffffff;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kmin = min(kmin, __shfl_xor(kmin, off, 64));
    kmax = max(kmax, __shfl_xor(kmax, off, 64));
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  kmin = red[0][0];
  kmax = red[1][0];
#pragma unroll
  for (int w2 = 1; w2 < kWaves; ++w2) {
    kmin = min(kmin, red[0][w2]);
    kmax = max(kmax, red[1][w2]);
  }

  f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[dt][i] = dvacc[dt][i] = 0.f;

  // staging: chunk idx = tid + kT * i of [tensor (Q, dO)][row][chunk]
  u32x4 sreg[SL];

  auto row_off = [&](int64_t row) -> int64_t {  // element offset of query row `row`
    const int64_t tk = row / grp;
    return (tk * p.hq + static_cast<int64_t>(g) * grp + row % grp) * D;
  };
  // metadata of the staged step, prefetched with the rows: threads < 32 hold their
  // row's lse / delta / interval, thread 32 the step's first block interval
  float m_lse = 0.f, m_dlt = 0.f;
  int m_lo = 0, m_hi = 0, m_uni = 0;
  auto load_step = [&](int64_t step) {
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int idx = tid + kT * i;
      if (SCH % kT == 0 || idx < SCH) {
        const int tensor = idx / (kStepRows * CPR), rem = idx % (kStepRows * CPR);
        const int64_t row = min(step * kStepRows + rem / CPR, R - 1);
        sreg[i] = *reinterpret_cast<const u32x4*>((tensor == 0 ? p.q : p.dout) + row_off(row) + 8 * (rem % CPR));
      }
    }
    if (tid < kStepRows) {
      const int64_t row_raw = step * kStepRows + tid;
      const bool rv = row_raw < R;
      const int64_t row = rv ? row_raw : R - 1;
      const int64_t tk = row / grp;
      const int bb = static_cast<int>(tk / kBlock);
      const int64_t li = tk * p.hq + static_cast<int64_t>(g) * grp + row % grp;
      const float ln = p.lse[li];
      m_lse = (rv && ln != -INFINITY) ? ln * kLog2e : INFINITY;
      m_dlt = p.delta[li];
      m_lo = self_tile ? kBlock * bb : p.sample_start[bb];
      m_hi = rv ? (self_tile ? kBlock * bb + kBlock : p.anchor[bb]) : -0x7fffffff;
    } else if (tid == kStepRows) {
      const int64_t r0 = step * kStepRows, r1 = r0 + kStepRows - 1;
      const int b0 = static_cast<int>(r0 / grp / kBlock);
      m_uni = r1 < R && static_cast<int>(r1 / grp / kBlock) == b0;
      m_lo = self_tile ? kBlock * b0 : p.sample_start[b0];
      m_hi = self_tile ? kBlock * b0 + kBlock : p.anchor[b0];
    }
  };
  auto store_step = [&](int b) {
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int idx = tid + kT * i;
      if (SCH % kT == 0 || idx < SCH) {
        const int tensor = idx / (kStepRows * CPR), rem = idx % (kStepRows * CPR);
        LdsTile<D>::store(stg[b][tensor], rem / CPR, rem % CPR, sreg[i]);
      }
    }
    if (tid < kStepRows) {
      meta[b].lse2[tid] = m_lse;
      meta[b].dlt[tid] = m_dlt;
      meta[b].lo[tid] = m_lo;
      meta[b].hi[tid] = m_hi;
    } else if (tid == kStepRows) {
      meta[b].uni = m_uni;
      meta[b].lo0 = m_lo;
      meta[b].hi0 = m_hi;
    }
  };

  auto step_hit = [&](int64_t st) -> bool {
    if (st >= n_steps) return false;
    const int64_t r0 = st * kStepRows;
    const int64_t r1 = min(r0 + kStepRows, R) - 1;
    const int b0 = static_cast<int>(r0 / grp / kBlock), b1 = static_cast<int>(r1 / grp / kBlock);
    bool hit = false;
    for (int b = b0; b <= b1; ++b) {
      const int lo = self_tile ? kBlock * b : p.sample_start[b];
      const int hi = self_tile ? kBlock * b + kBlock : p.anchor[b];
      hit |= (lo <= kmax) && (hi > kmin);
    }
    return hit;
  };

  // Count the steps that reach this tile and split them over `parts` workgroups
  // (interleaved), so that heavily read key tiles do not set the kernel's length.
  int n_hit = 0;
  for (int64_t base = 0; base < n_steps; base += kT) n_hit += __syncthreads_count(step_hit(base + tid));
  const bool can_split = p.ws_parts != nullptr && !self_tile;
  const int parts = can_split ? max(1, min(kMaxParts, (n_hit + kStepsPerPart - 1) / kStepsPerPart)) : 1;
  if (part >= parts) return;
  if (can_split && part == 0 && tid == 0) p.ws_parts[tile * p.hkv + g] = parts;

  // V rows of the workgroup's keys -> LDS (row-major, chunk ^ (row & 7))
  for (int idx = tid; idx < kKeysPerWG * CPR; idx += kT) {
    const int row = idx / CPR, j = idx % CPR;
    const int64_t src_row = min(krow0 + row, key_rows - 1);
    LdsTile<D>::store(vtile, row, j, *reinterpret_cast<const u32x4*>(V + (src_row * p.hkv + g) * D + 8 * j));
  }
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(K + (krc * p.hkv + g) * D + 16 * ks + 8 * h2));

  int seen = 0;  // hits in earlier batches
  for (int64_t base = 0; base < n_steps; base += kT) {
    // compact this part's share of the batch's hits (global hit index % parts == part)
    const bool hit = step_hit(base + tid);
    const uint64_t mask = __ballot(hit);
    if (lane == 0) wave_cnt[wave] = __popcll(mask);
    __syncthreads();
    int pre = 0, total_b = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const int c = wave_cnt[w2];
      pre += w2 < wave ? c : 0;
      total_b += c;
    }
    const int gidx = seen + pre + __popcll(mask & ((uint64_t{1} << lane) - 1));
    // entries of this part: gidx = part + parts * j  ->  list slot j - first_j
    const int first_j = (seen - part + parts - 1) / parts;  // first j with part + parts*j >= seen
    if (hit && (gidx - part) % parts == 0) step_list[(gidx - part) / parts - first_j] = static_cast<int>(base + tid);
    const int last_excl = seen + total_b;  // hits [seen, last_excl) are in this batch
    const int end_j = (last_excl - part + parts - 1) / parts;
    const int total = max(0, end_j - first_j);
    seen = last_excl;
    __syncthreads();
    if (total == 0) continue;

    load_step(step_list[0]);
    store_step(0);
    __syncthreads();
    int buf = 0;
    for (int si = 0; si < total; ++si) {
      const bool has_next = si + 1 < total;
      if (has_next) load_step(step_list[si + 1]);

      const StepMeta& mt = meta[buf];
      // wave-uniform step facts in scalar registers
      const bool uni = __builtin_amdgcn_readfirstlane(mt.uni) != 0;
      const int lo0 = __builtin_amdgcn_readfirstlane(mt.lo0);
      const int hi0 = __builtin_amdgcn_readfirstlane(mt.hi0);
      const bool lane_ok = kvalid && kcoord >= lo0 && kcoord < hi0;
      bool run = true, all_ok = false;
      if (uni) {
        run = __any(lane_ok);
        all_ok = __all(lane_ok);
      }
      if (run) {
        const uint16_t* lq = stg[buf][0];
        const uint16_t* ld = stg[buf][1];
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 qa = LdsTile<D>::frag(lq, l32, 2 * ks + h2);
          const bf16x8 da = LdsTile<D>::frag(ld, l32, 2 * ks + h2);
          const bf16x8 vb = LdsTile<D>::frag(vtile, krow, 2 * ks + h2);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vb, pacc, 0, 0, 0);
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // rows 8j + 4h2 + 0..3 of the step
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&mt.lse2[8 * j + 4 * h2]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&mt.dlt[8 * j + 4 * h2]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * j + i;
            float pr = __builtin_amdgcn_exp2f(fmaf(sacc[r], p.scale_log2, -l4[i]));
            if (!all_ok) {
              if (uni) {
                pr = lane_ok ? pr : 0.f;
              } else {
                const int row = 8 * j + 4 * h2 + i;
                if (!(kvalid && kcoord >= mt.lo[row] && kcoord < mt.hi[row])) pr = 0.f;
              }
            }
            const float ds = pr * (pacc[r] - d4[i]);
            pb[r / 8][r % 8] = static_cast<__bf16>(pr);
            sb[r / 8][r % 8] = static_cast<__bf16>(ds);
          }
        }
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int sl = lane & 15, col = 32 * dt + 16 * ((lane >> 4) & 1);
            const bf16x8 dta = LdsTile<D>::frag_t(ld, tr_row_a(kq, h2, sl), tr_row_b(kq, h2, sl), col, sl);
            const bf16x8 qta = LdsTile<D>::frag_t(lq, tr_row_a(kq, h2, sl), tr_row_b(kq, h2, sl), col, sl);
            dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta, pb[kq], dvacc[dt], 0, 0, 0);
            dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, sb[kq], dkacc[dt], 0, 0, 0);
          }
        }
      }

      if (has_next) store_step(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  if (!kvalid) return;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dcol = 32 * dt + 8 * jj + 4 * h2;
      const f32x4 kv4 = f32x4{dkacc[dt][4 * jj], dkacc[dt][4 * jj + 1], dkacc[dt][4 * jj + 2], dkacc[dt][4 * jj + 3]};
      const f32x4 vv4 = f32x4{dvacc[dt][4 * jj], dvacc[dt][4 * jj + 1], dvacc[dt][4 * jj + 2], dvacc[dt][4 * jj + 3]};
      if (parts == 1) {
        float* dK = self_tile ? p.dk_self : p.dk;
        float* dV = self_tile ? p.dv_self : p.dv;
        const int64_t o = (kr * p.hkv + g) * D + dcol;
        *reinterpret_cast<f32x4*>(dK + o) = kv4 * p.scale;
        *reinterpret_cast<f32x4*>(dV + o) = vv4;
      } else {  // partial sums of this part: added up by the reduce pass
        float* slot = p.ws_slots + ((static_cast<int64_t>(tile) * p.hkv + g) * kMaxParts + part) *
                                       (static_cast<int64_t>(kKeysPerWG) * 2 * D);
        *reinterpret_cast<f32x4*>(slot + (krow * 2 + 0) * D + dcol) = kv4;
        *reinterpret_cast<f32x4*>(slot + (krow * 2 + 1) * D + dcol) = vv4;
      }
    }
}

// Sum of the partial dK/dV of split context tiles (one workgroup per tile and kv head).
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(BwdParams p) {
  const int g = blockIdx.x % p.hkv;
  const int tile = blockIdx.x / p.hkv;
  const int parts = p.ws_parts[tile * p.hkv + g];
  if (parts <= 1) return;
  const int64_t slot_elems = static_cast<int64_t>(kKeysPerWG) * 2 * D;
  const float* slots = p.ws_slots + (static_cast<int64_t>(tile) * p.hkv + g) * kMaxParts * slot_elems;
  const int64_t krow0 = static_cast<int64_t>(tile) * kKeysPerWG;
  constexpr int V4 = kKeysPerWG * 2 * D / 4;
  for (int i = threadIdx.x; i < V4; i += 256) {
    const int e = 4 * i;
    const int krow = e / (2 * D), which = (e / D) % 2, dcol = e % D;
    const int64_t kr = krow0 + krow;
    if (kr >= p.n_loc) continue;
    f32x4 acc = *reinterpret_cast<const f32x4*>(slots + e);
    for (int q = 1; q < parts; ++q) acc += *reinterpret_cast<const f32x4*>(slots + q * slot_elems + e);
    float* dst = (which == 0 ? p.dk : p.dv) + (kr * p.hkv + g) * D + dcol;
    *reinterpret_cast<f32x4*>(dst) = which == 0 ? acc * p.scale : acc;
  }
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
  p.dk = static_cast<float*>(a.dk);
  p.dv = static_cast<float*>(a.dv);
  p.dk_self = static_cast<float*>(a.dk_self);
  p.dv_self = static_cast<float*>(a.dv_self);
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
  p.ws_parts = nullptr;
  p.ws_slots = nullptr;
  if (a.flags & SXA_BWD_DQ) {
    const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * (a.hq / a.hkv);
    const int64_t n_dq = (rows + 32 * kDqWaves - 1) / (32 * kDqWaves) * a.hkv;
    dq_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_dq)), dim3(64 * kDqWaves), 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!(a.flags & SXA_BWD_DKDV)) return hipSuccess;
  const int64_t n_ctx_tiles = (a.n_loc + kKeysPerWG - 1) / kKeysPerWG;
  const int64_t n_q = static_cast<int64_t>(a.n_blk) * kBlock;
  const int64_t n_self_tiles = a.k_self ? (n_q + kKeysPerWG - 1) / kKeysPerWG : 0;
  const int64_t n_tiles = n_ctx_tiles + n_self_tiles;
  if (n_tiles == 0) return hipSuccess;
  const bool split = a.workspace != nullptr;
  if (split) {
    p.ws_parts = static_cast<int32_t*>(a.workspace);
    p.ws_slots = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                          ((n_ctx_tiles * a.hkv * 4 + 255) / 256) * 256);
  }
  const int64_t n_kv = n_tiles * a.hkv * (split ? kMaxParts : 1);
  dkdv_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_kv)), dim3(64 * kKvWaves), 0, s>>>(p, static_cast<int>(n_ctx_tiles),
                                                                            static_cast<int>(n_tiles));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (split && n_ctx_tiles > 0) {
    dkdv_reduce_kernel<D><<<dim3(static_cast<unsigned>(n_ctx_tiles * a.hkv)), dim3(256), 0, s>>>(p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

int64_t bwd_workspace_bytes(int64_t n_loc, int32_t hkv, int32_t d) {
  const int64_t tiles = (n_loc + kKeysPerWG - 1) / kKeysPerWG;
  return ((tiles * hkv * 4 + 255) / 256) * 256 +
         tiles * hkv * kMaxParts * static_cast<int64_t>(kKeysPerWG) * 2 * d * 4;
}

hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace sxa
