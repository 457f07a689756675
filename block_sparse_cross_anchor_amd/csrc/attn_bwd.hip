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

namespace sxa {
namespace {

constexpr int kTileKeys = 64;
constexpr int kWaves = 8;
constexpr int kT = 64 * kWaves;

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
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dk_self;
  uint16_t* dv_self;
  const int32_t* anchor;
  const int32_t* sample_start;
  const int32_t* chunk_gstart;
  const int32_t* chunk_len;
  int64_t n_loc;
  int32_t n_blk, hq, hkv, n_chunk;
  float scale;
  float scale_log2;  // scale * log2(e)
  int32_t dq_overwrite;
};

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// position of index i inside a 16-aligned group when bits 2 and 3 are swapped:
// the order in which one lane holds MFMA accumulator rows 8*(r/4) + 4h + r%4
__device__ __forceinline__ int perm23(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}
__device__ __forceinline__ int swz64(int d) { return (d & 7) ^ ((d >> 3) & 7); }

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

// K tile: row-major (16-byte chunks XOR (key & 7)) and transposed (64 keys per
// head-dim row, keys permuted by perm23, chunks XOR swz64(d)); V tile row-major.
template <int D>
struct DqTileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int KIT = kTileKeys / 2 * CPR;  // (key pair, chunk) items
  static constexpr int VCH = kTileKeys * CPR;      // V chunks
  static constexpr int KL = (KIT + kT - 1) / kT;
  static constexpr int VL = (VCH + kT - 1) / kT;
  u32x4 k[KL][2];
  u32x4 v[VL];

  __device__ __forceinline__ void load(const Tile& t, const BwdParams& p, int g, int tid) {
    const uint16_t* K = t.self ? p.k_self : p.k;
    const uint16_t* V = t.self ? p.v_self : p.v;
    const int last = t.nrows - 1;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int it = tid + kT * i;
      if (KIT % kT == 0 || it < KIT) {
        const int q2 = it / CPR, j = it % CPR;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int key = min(2 * q2 + kk, last);
          k[i][kk] = *reinterpret_cast<const u32x4*>(K + ((t.row0 + key) * p.hkv + g) * D + 8 * j);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int idx = tid + kT * i;
      if (VCH % kT == 0 || idx < VCH) {
        const int key = min(idx / CPR, last), j = idx % CPR;
        v[i] = *reinterpret_cast<const u32x4*>(V + ((t.row0 + key) * p.hkv + g) * D + 8 * j);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lk, uint16_t* lkt, uint16_t* lv, int tid) const {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int it = tid + kT * i;
      if (KIT % kT == 0 || it < KIT) {
        const int q2 = it / CPR, j = it % CPR;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int key = 2 * q2 + kk;
          *reinterpret_cast<u32x4*>(lk + key * D + 8 * (j ^ (key & 7))) = k[i][kk];
        }
        const int pos = perm23(2 * q2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * j + e;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w = __builtin_amdgcn_perm(k[i][1][e >> 1], k[i][0][e >> 1], sel);
          const int phys = (pos >> 3) ^ swz64(d);
          *reinterpret_cast<uint32_t*>(lkt + d * kTileKeys + 8 * phys + (pos & 7)) = w;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int idx = tid + kT * i;
      if (VCH % kT == 0 || idx < VCH) {
        const int key = idx / CPR, j = idx % CPR;
        *reinterpret_cast<u32x4*>(lv + key * D + 8 * (j ^ (key & 7))) = v[i];
      }
    }
  }
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kT, kT))) void dq_bf16_kernel(BwdParams p) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int ROWS = 32 * kWaves;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][3][kTileKeys * D];

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

  DqTileRegs<D> regs;
  regs.load(cur, p, g, tid);
  regs.store(lds[0][0], lds[0][1], lds[0][2], tid);
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
      const uint16_t* lkt = lds[buf][1];
      const uint16_t* lv = lds[buf][2];
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[mt][i] = pacc[mt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int key = 32 * mt + l32;
          const int off = key * D + 8 * ((2 * ks + h2) ^ (key & 7));
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lk + off));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lv + off));
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
          const int d = 32 * dt + l32;
          const bf16x8 kt = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(lkt + d * kTileKeys + 8 * ((2 * kq + h2) ^ swz64(d))));
          dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf[kq], dqacc[dt], 0, 0, 0);
        }
      }
    }

    if (has_next) regs.store(lds[buf ^ 1][0], lds[buf ^ 1][1], lds[buf ^ 1][2], tid);
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
// context rows, or own-block rows for the tiles after the context ones).  Query
// rows of kv head g are numbered r = token * grp + (h - g*grp) and visited in
// steps of 32.  A step is visited when one of its blocks' key intervals meets
// the workgroup's keys (for own-block tiles: when it holds one of their blocks).

constexpr int kKeysPerWG = 32 * kWaves;
constexpr int kStepRows = 32;

struct StepLds {
  int lo[kStepRows];   // per row: allowed key interval [lo, hi) in key coordinates
  int hi[kStepRows];
  float lse2[kStepRows];
  float dlt[kStepRows];
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kT, kT))) void dkdv_bf16_kernel(BwdParams p,
                                                                                      int n_ctx_tiles) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = D / 8;
  // per stage: Q row-major, Q^T, dO row-major, dO^T (32 rows each)
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][4][kStepRows * D];
  __shared__ StepLds meta[2];
  __shared__ int step_list[kT];
  __shared__ int wave_cnt[kWaves];
  __shared__ int red[2][kWaves];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  const int g = blockIdx.x % p.hkv;
  const int tile = blockIdx.x / p.hkv;
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
  const int64_t kr = krow0 + 32 * wave + l32;
  const bool kvalid = kr < key_rows;
  const int64_t krc = kvalid ? kr : key_rows - 1;
  int kcoord;  // global position (context) or own-block row (self)
  if (self_tile) {
    kcoord = static_cast<int>(krc);
  } else {
    int64_t off = 0;
    kcoord = 0;
    for (int c = 0; c < p.n_chunk; ++c) {
      const int len = p.chunk_len[c];
      if (krc < off + len) {
        kcoord = p.chunk_gstart[c] + static_cast<int>(krc - off);
        break;
      }
      off += len;
    }
  }
  const int kc_min_lane = kvalid ? kcoord : 0x7fffffff;
  const int kc_max_lane = kvalid ? kcoord : -0x7fffffff;

  // K and V of this lane's key as MFMA B operands (8 head-dim values per k-step)
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(K + (krc * p.hkv + g) * D + 16 * ks + 8 * h2));
    vf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(V + (krc * p.hkv + g) * D + 16 * ks + 8 * h2));
  }

  // key-coordinate range of the workgroup
  int kmin = kc_min_lane, kmax = kc_max_lane;
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

  // step staging: thread -> (row pair, chunk) of Q (first half of threads) or dO
  constexpr int ITEMS = kStepRows / 2 * CPR;  // per tensor
  static_assert(2 * ITEMS <= kT, "one item per thread");
  const bool is_do = tid >= ITEMS;
  const int item = is_do ? tid - ITEMS : tid;
  const bool has_item = tid < 2 * ITEMS;
  const int ipair = item / CPR, ichunk = item % CPR;

  auto step_row = [&](int64_t step, int i) -> int64_t { return step * kStepRows + i; };
  auto row_gaddr = [&](int64_t row) -> int64_t {  // element offset of query row `row`
    const int64_t tk = row / grp;
    return (tk * p.hq + static_cast<int64_t>(g) * grp + row % grp) * D;
  };

  u32x4 sreg[2];
  auto load_step = [&](int64_t step) {
    if (has_item) {
      const uint16_t* src = is_do ? p.dout : p.q;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int64_t row = min(step_row(step, 2 * ipair + kk), R - 1);
        sreg[kk] = *reinterpret_cast<const u32x4*>(src + row_gaddr(row) + 8 * ichunk);
      }
    }
  };
  auto store_step = [&](int64_t step, int b) {
    if (has_item) {
      uint16_t* rm = lds[b][is_do ? 2 : 0];
      uint16_t* tr = lds[b][is_do ? 3 : 1];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = 2 * ipair + kk;
        *reinterpret_cast<u32x4*>(rm + row * D + 8 * (ichunk ^ (row & 7))) = sreg[kk];
      }
      const int pos = perm23(2 * ipair);  // 32 rows: bit 4 kept
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * ichunk + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t w = __builtin_amdgcn_perm(sreg[1][e >> 1], sreg[0][e >> 1], sel);
        const int phys = (pos >> 3) ^ ((d >> 1) & 3);
        *reinterpret_cast<uint32_t*>(tr + d * kStepRows + 8 * phys + (pos & 7)) = w;
      }
    }
    if (tid < kStepRows) {
      const int64_t row_raw = step_row(step, tid);
      const bool rv = row_raw < R;
      const int64_t row = rv ? row_raw : R - 1;
      const int64_t tk = row / grp;
      const int bb = static_cast<int>(tk / kBlock);
      const int64_t li = tk * p.hq + static_cast<int64_t>(g) * grp + row % grp;
      const float ln = p.lse[li];
      meta[b].lse2[tid] = (rv && ln != -INFINITY) ? ln * kLog2e : INFINITY;
      meta[b].dlt[tid] = p.delta[li];
      meta[b].lo[tid] = self_tile ? kBlock * bb : p.sample_start[bb];
      meta[b].hi[tid] = rv ? (self_tile ? kBlock * bb + kBlock : p.anchor[bb]) : -0x7fffffff;
    }
  };

  // does a step hold a row whose block can read a key of this workgroup?
  auto step_hits = [&](int64_t step) -> bool {
    const int64_t r0 = step * kStepRows;
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

  int buf = 0;
  bool primed = false;
  for (int64_t base = 0; base < n_steps; base += kT) {
    // compact the steps of this batch that can touch the workgroup's keys
    const int64_t st = base + tid;
    const bool hit = st < n_steps && step_hits(st);
    const uint64_t mask = __ballot(hit);
    if (lane == 0) wave_cnt[wave] = __popcll(mask);
    __syncthreads();
    int pre = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const int c = wave_cnt[w2];
      pre += w2 < wave ? c : 0;
      total += c;
    }
    if (hit) step_list[pre + __popcll(mask & ((uint64_t{1} << lane) - 1))] = static_cast<int>(st);
    __syncthreads();
    if (total == 0) continue;

    if (!primed) {
      load_step(step_list[0]);
      store_step(step_list[0], 0);
      __syncthreads();
      primed = true;
      buf = 0;
    }
    for (int si = 0; si < total; ++si) {
      const bool has_next = si + 1 < total;
      if (has_next) load_step(step_list[si + 1]);

      // ---- this wave: 32 rows x 32 keys
      const StepLds& mt = meta[buf];
      // per-register rows 8*(i/4) + 4*h2 + i%4 of the step
      bool allowed[16];
      bool any = false, all = true;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i / 4) + 4 * h2 + (i % 4);
        allowed[i] = kvalid && kcoord >= mt.lo[row] && kcoord < mt.hi[row];
        any |= allowed[i];
        all &= allowed[i];
      }
      if (__any(any)) {
        const bool all_ok = __all(all);
        const uint16_t* lq = lds[buf][0];
        const uint16_t* lqt = lds[buf][1];
        const uint16_t* ld = lds[buf][2];
        const uint16_t* ldt = lds[buf][3];
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = l32 * D + 8 * ((2 * ks + h2) ^ (l32 & 7));
          const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lq + off));
          const bf16x8 da = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ld + off));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ks], pacc, 0, 0, 0);
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 8 * (i / 4) + 4 * h2 + (i % 4);
          float pr = __builtin_amdgcn_exp2f(fmaf(sacc[i], p.scale_log2, -mt.lse2[row]));
          if (!all_ok && !allowed[i]) pr = 0.f;
          const float ds = pr * (pacc[i] - mt.dlt[row]);
          pb[i / 8][i % 8] = static_cast<__bf16>(pr);
          sb[i / 8][i % 8] = static_cast<__bf16>(ds);
        }
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int d = 32 * dt + l32;
            const int off = d * kStepRows + 8 * ((2 * kq + h2) ^ ((d >> 1) & 3));
            const bf16x8 dta = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ldt + off));
            const bf16x8 qta = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lqt + off));
            dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dta, pb[kq], dvacc[dt], 0, 0, 0);
            dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qta, sb[kq], dkacc[dt], 0, 0, 0);
          }
        }
      }

      if (has_next) store_step(step_list[si + 1], buf ^ 1);
      __syncthreads();
      if (has_next) buf ^= 1;
    }
    // the next batch restages from its first step
    primed = false;
  }

  if (!kvalid) return;
  uint16_t* dK = self_tile ? p.dk_self : p.dk;
  uint16_t* dV = self_tile ? p.dv_self : p.dv;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t o = (kr * p.hkv + g) * D + 32 * dt + 8 * jj + 4 * h2;
      *reinterpret_cast<u32x2*>(dK + o) =
          u32x2{pack_bf16x2(p.scale * dkacc[dt][4 * jj], p.scale * dkacc[dt][4 * jj + 1]),
                pack_bf16x2(p.scale * dkacc[dt][4 * jj + 2], p.scale * dkacc[dt][4 * jj + 3])};
      *reinterpret_cast<u32x2*>(dV + o) = u32x2{pack_bf16x2(dvacc[dt][4 * jj], dvacc[dt][4 * jj + 1]),
                                                pack_bf16x2(dvacc[dt][4 * jj + 2], dvacc[dt][4 * jj + 3])};
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
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.dk_self = static_cast<uint16_t*>(a.dk_self);
  p.dv_self = static_cast<uint16_t*>(a.dv_self);
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
  if (a.flags & SXA_BWD_DQ) {
    const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * (a.hq / a.hkv);
    const int64_t n_dq = (rows + 32 * kWaves - 1) / (32 * kWaves) * a.hkv;
    dq_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_dq)), dim3(kT), 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!(a.flags & SXA_BWD_DKDV)) return hipSuccess;
  const int64_t n_ctx_tiles = (a.n_loc + kKeysPerWG - 1) / kKeysPerWG;
  const int64_t n_self_tiles =
      a.k_self ? (static_cast<int64_t>(a.n_blk) * kBlock + kKeysPerWG - 1) / kKeysPerWG : 0;
  const int64_t n_kv = (n_ctx_tiles + n_self_tiles) * a.hkv;
  if (n_kv == 0) return hipSuccess;
  dkdv_bf16_kernel<D><<<dim3(static_cast<unsigned>(n_kv)), dim3(kT), 0, s>>>(p, static_cast<int>(n_ctx_tiles));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const AttnArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace sxa
