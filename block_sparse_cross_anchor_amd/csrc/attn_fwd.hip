// bf16 forward of the anchor-masked block-sparse cross-attention on gfx950 MFMA.
//
// What is computed ("Split-KV speeds diffusion drafter training...", sections
// "Why short queries change the problem" and "Exchange the smaller side"): for
// every query row (token i of block b, head h) the softmax over the allowed keys
// of this call -- context positions [sample_start[b], anchor[b]) inside the local
// chunks, plus the 16 own-block keys when k_self is given -- giving the partial
// output O and its natural-log log-sum-exp, from which partials merge exactly.
//
// Work decomposition
//   * Rows of one kv head g: r = token * grp + (h - g*grp), grp = hq / hkv.  With
//     grp = 4 the 64 rows of one wave are one block's 16 tokens x 4 heads, which
//     share one mask.  A workgroup (4 waves) owns 256 consecutive rows of one kv
//     head: for grp = 4 that is 4 consecutive blocks, normally of one sample, so
//     their key intervals start at the same position and K/V tiles are shared
//     through LDS.
//   * Linear workgroup id L -> (kv head L % hkv, row group L / hkv): consecutive
//     ids are dispatched round-robin over the 8 XCDs, so with hkv = 8 each XCD
//     serves one kv head and its K/V stays in that XCD's L2.
//   * Keys are visited in tiles of 64 rows: first the own-block rows of the
//     workgroup's blocks, then, chunk by chunk, the tiles (aligned to the chunk
//     start) that meet the union of the workgroup's intervals.  Each wave skips
//     the MFMAs of tiles outside all of its rows' intervals (anchor-driven tile
//     skipping) and masks only tiles that are partially allowed.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16; lane l, half h = l / 32):
//   S^T = K Q^T   A = K tile rows (from LDS), B = Q^T (registers, whole kernel)
//                 result lane l holds column (query row) l % 32 and keys
//                 8*(r/4) + 4h + r%4 of the 32-key M tile.
//   O^T += V^T P^T with P^T taken straight from the S^T registers (converted to
//                 bf16); the A operand V^T is read from the row-major V tile with
//                 the transposing LDS read (two ds_read_b64_tr_b16 per fragment),
//                 in the key order the S^T registers hold.
//   Row max needs one exchange between the two lane halves; row sums are kept
//   per half and added once at the end.
//   Both LDS tiles are row-major, XOR-swizzled in 16-byte units (lds_tile.h).
// Online softmax in base 2: x = s * scale * log2(e); p = exp2(x - m).
#include "device_common.h"
#include "internal.h"
#include "kv_walk.h"
#include "lds_tile.h"


namespace sxa {
namespace {

constexpr float kRescaleSlack = 8.f;  // log2 units
#ifndef SXA_FWD_KPF
#define SXA_FWD_KPF 1
#endif
constexpr int KPF = SXA_FWD_KPF;  // k-steps between a K fragment's LDS read and its MFMA


struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_self;
  const uint16_t* v_self;
  const int32_t* anchor;
  const int32_t* sample_start;
  const int32_t* chunk_gstart;
  const int32_t* chunk_len;
  void* o;
  float* lse;
  const int32_t* rg_order;  // row group of workgroup blockIdx / hkv (nullptr: identity)
  // split forward (jobs != nullptr): job blockIdx / hkv = {row group, first tile, end
  // tile, slot}; a job with a slot writes its partial O and lse there
  const int4* jobs;
  float* part_o;
  float* part_lse;
  int32_t n_blk, hq, hkv, n_chunk;
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// NT: 32-row N tiles per wave (rows per wave = 32 * NT); WAVES: waves per workgroup.
template <int D, int NT, int WAVES, int NSTAGE, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES))) void
fwd_bf16_kernel(FwdParams p) {
  static_assert(NSTAGE == 2 || NSTAGE == 3, "two or three tile buffers");
  constexpr int ROWS = 32 * NT * WAVES;  // rows per workgroup
  constexpr int KS = D / 16;             // k-steps of S^T
  constexpr int DT = D / 32;             // 32-row d tiles of O^T
  using Dma = TileDma<D, WAVES, true>;
  __shared__ __attribute__((aligned(256))) uint16_t bufs[NSTAGE][Dma::ELEMS];

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64, h2 = lane / 32, l32 = lane % 32;
  const int g = blockIdx.x % p.hkv;
  int wg, t_skip = 0, t_left = 0x7fffffff;
  if (p.jobs) {
    const int4 jb = p.jobs[blockIdx.x / p.hkv];
    if (jb.x < 0) return;  // more job slots than jobs
    wg = jb.x;
    t_skip = jb.y;
    t_left = jb.z - jb.y;
  } else {
    wg = p.rg_order ? p.rg_order[blockIdx.x / p.hkv] : static_cast<int>(blockIdx.x / p.hkv);
  }
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
  w.start(p.k_self != nullptr, b_first, b_last);
  // a piece of a split row group: skip to its first tile, stop after its last
  Tile skipped;
  for (int i = 0; i < t_skip; ++i) walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, skipped);
  auto next_tile = [&](Tile& t) {
    if (t_left == 0) return false;
    --t_left;
    return walk_next(w, p.chunk_gstart, p.chunk_len, p.n_chunk, LO, HI, t);
  };

  float m[NT], l[NT];
  f32x16 oacc[DT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][nt][r] = 0.f;
  }

  Tile cur;
  const bool have = next_tile(cur);
  if (!have) {  // no allowed key in this call: O = 0, lse = -inf
    const int slot = p.jobs ? p.jobs[blockIdx.x / p.hkv].w : -1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int lr = 32 * NT * wave + 32 * nt + l32;
      const int64_t r = wg_row0 + lr;
      if (slot >= 0) {
        const int64_t pr = (static_cast<int64_t>(slot) * p.hkv + g) * ROWS + lr;
        if (h2 == 0) p.part_lse[pr] = -INFINITY;
        for (int d0 = h2 * (D / 2); d0 < (h2 + 1) * (D / 2); d0 += 4)
          *reinterpret_cast<f32x4*>(p.part_o + pr * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
        continue;
      }
      if (r >= R) continue;
      const int64_t tok = r / grp;
      const int64_t orow = tok * p.hq + static_cast<int64_t>(g) * grp + static_cast<int>(r % grp);
      if (h2 == 0) p.lse[orow] = -INFINITY;
#pragma unroll
      for (int d0 = h2 * (D / 2); d0 < (h2 + 1) * (D / 2); d0 += 8) {
        if constexpr (OUT_BF16)
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.o) + orow * D + d0) = u32x4{0, 0, 0, 0};
        else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + orow * D + d0) = f32x4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + orow * D + d0 + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    return;
  }

  // per-lane query columns (one per 32-row N tile)
  int clo[NT], chi[NT], slo[NT], shi[NT];
  int64_t orow[NT];
  bool valid[NT];
  bf16x8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t r = wg_row0 + 32 * NT * wave + 32 * nt + l32;
    valid[nt] = r < R;
    const int64_t rr = valid[nt] ? r : 0;
    const int64_t tok = rr / grp;
    const int hh = static_cast<int>(rr % grp);
    const int blk = static_cast<int>(tok / kBlock);
    clo[nt] = valid[nt] ? p.sample_start[blk] : 0;
    chi[nt] = valid[nt] ? p.anchor[blk] : 0;
    slo[nt] = valid[nt] ? kBlock * blk : 0;
    shi[nt] = valid[nt] ? kBlock * blk + kBlock : 0;
    orow[nt] = tok * p.hq + static_cast<int64_t>(g) * grp + hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(p.q + orow[nt] * D + 16 * ks + 8 * h2);
      qf[nt][ks] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // Three-stage pipeline: tile t is computed from buffer t % 3 while the DMA of
  // tiles t + 1 and t + 2 is in flight.  The prologue's own loads complete first,
  // so that the only vector-memory operations in flight in the loop are the DMA.
  wait_vmcnt<0>();
  // LDS byte offsets within a tile buffer (see LdsTile): K rows 32 mt + l32, and the
  // transposed V reads of the key steps
  int f_k = LdsTile<D>::frag_off(l32, h2);
  int t_a = LdsTile<D>::tr_off(4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
  int t_b = LdsTile<D>::tr_off(8 + 4 * h2 + ((lane & 15) >> 2), (lane >> 4) & 1, lane & 15);
  constexpr uint32_t kVOff = kTileKeys * D * 2;  // V rows follow the K rows
  Tile n1, n2;
  const Dma dma(p.hkv, wave, lane);
  dma.issue(cur, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[0]));
  bool have1 = false;
  if constexpr (NSTAGE == 3) {
    have1 = next_tile(n1);
    if (have1) dma.issue(n1, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[1]));
  }
  int cb = 0;
  while (true) {
    bool have2 = false;
    if constexpr (NSTAGE == 3) {
      if (have1) wait_vmcnt<Dma::NI>();  // this wave's DMA of `cur` done (n1 may be in flight)
      else wait_vmcnt<0>();
      barrier_nofence();                 // ... and every wave's; all reads of the third buffer are done
      have2 = next_tile(n2);  // false once exhausted
      if (have2) dma.issue(n2, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[cb == 0 ? 2 : cb - 1]));
    } else {
      wait_vmcnt<0>();
      barrier_nofence();  // `cur` landed everywhere; the other buffer is no longer read
      have1 = next_tile(n1);
      if (have1) dma.issue(n1, p.k, p.v, p.k_self, p.v_self, p.hkv, g, lane, lds_addr(bufs[cb ^ 1]));
    }
      // per-lane constants are redefined opaquely per tile so that derived addresses
      // are recomputed rather than held
      asm volatile("" : "+v"(f_k), "+v"(t_a), "+v"(t_b));
      // ---- this wave's share of the tile
      int a_lo[NT], a_hi[NT];
      bool any = false, full = true;
  #pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int lo = cur.self ? slo[nt] : clo[nt];
        const int hi = cur.self ? shi[nt] : chi[nt];
        a_lo[nt] = max(lo - cur.coord0, 0);
        a_hi[nt] = min(hi - cur.coord0, cur.nrows);
        any |= a_lo[nt] < a_hi[nt];
        full &= (a_lo[nt] == 0) & (a_hi[nt] == kTileKeys);
      }
      if (__any(any)) {
        const bool all_full = __all(full);
        const uint32_t base = lds_addr(bufs[cb]);
        const uint32_t kb = base + f_k, ta = base + t_a + kVOff, tb = base + t_b + kVOff;
        f32x16 sacc[2][NT];
  #pragma unroll
        for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
          for (int nt = 0; nt < NT; ++nt)
  #pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mt][nt][r] = 0.f;
        // K fragments are read KPF k-steps ahead of their MFMAs, so the LDS latency
        // is covered by the MFMAs in between
        bf16x8 kf[KPF + 1][2];
  #pragma unroll
        for (int ks = 0; ks < KPF; ++ks)
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt) kf[ks][mt] = lds_frag((kb ^ (32 * ks)) + mt * 64 * D);
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + KPF < KS) {
  #pragma unroll
            for (int mt = 0; mt < 2; ++mt)
              kf[(ks + KPF) % (KPF + 1)][mt] = lds_frag((kb ^ (32 * (ks + KPF))) + mt * 64 * D);
          }
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              sacc[mt][nt] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % (KPF + 1)][mt], qf[nt][ks], sacc[mt][nt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pf[NT][4];
        bool need[NT];
        float tmax[NT];
        bool any_need = false;
  #pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (!all_full) {
            // key = c + 4 h2 with c a compile-time constant: compare c against the
            // bounds shifted by 4 h2, so no per-element key is held in a register
            const int lo = a_lo[nt] - 4 * h2, hi = a_hi[nt] - 4 * h2;
  #pragma unroll
            for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int c = 32 * mt + 8 * (r / 4) + (r % 4);
                if (c < lo || c >= hi) sacc[mt][nt][r] = -INFINITY;
              }
          }
          float mx = -INFINITY;
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][nt][r]);
          mx = fmaxf(mx, swap_halves(mx)) * p.scale_log2;
          need[nt] = mx > m[nt] + kRescaleSlack;
          tmax[nt] = mx;
          any_need |= need[nt];
        }
        // Lazy rescale: the running max of a column only moves when the tile max
        // exceeds it by more than kRescaleSlack (so p <= 2^kRescaleSlack); the O
        // accumulators are rescaled only then, for the whole wave at once.
        if (__any(any_need)) {
  #pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float mnew = need[nt] ? tmax[nt] : m[nt];
            const float alpha =
                need[nt] ? (m[nt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[nt] - mnew)) : 1.f;
            m[nt] = mnew;
            l[nt] *= alpha;
  #pragma unroll
            for (int dt = 0; dt < DT; ++dt)
  #pragma unroll
              for (int r = 0; r < 16; ++r) oacc[dt][nt][r] *= alpha;
          }
        }
  #pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float muse = m[nt] == -INFINITY ? 0.f : m[nt];
          float rs = 0.f;
  #pragma unroll
          for (int mt = 0; mt < 2; ++mt)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mt][nt][r], p.scale_log2, -muse));
              sacc[mt][nt][r] = e;
              rs += e;
            }
          l[nt] += rs;
  #pragma unroll
          for (int kq = 0; kq < 4; ++kq)
  #pragma unroll
            for (int i = 0; i < 8; ++i)
              pf[nt][kq][i] = static_cast<__bf16>(sacc[kq / 2][nt][8 * (kq % 2) + i]);
        }
  #pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
  #pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 vf = lds_frag_t((ta ^ (64 * dt)) + kq * 32 * D, (tb ^ (64 * dt)) + kq * 32 * D);
  #pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[nt][kq], oacc[dt][nt], 0, 0, 0);
          }
        }
      }


    if (!have1) break;
    cur = n1;
    if constexpr (NSTAGE == 3) {
      n1 = n2;
      have1 = have2;
      cb = cb == 2 ? 0 : cb + 1;
    } else {
      cb ^= 1;
    }
  }

  // ---- epilogue: normalise, write O and lse (a piece: its slot, float32)
  const int slot = p.jobs ? p.jobs[blockIdx.x / p.hkv].w : -1;
  if (slot >= 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = l[nt] + swap_halves(l[nt]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t pr = (static_cast<int64_t>(slot) * p.hkv + g) * ROWS + 32 * NT * wave + 32 * nt + l32;
      if (h2 == 0) p.part_lse[pr] = lt > 0.f ? (m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * dt + 8 * jj + 4 * h2;
          *reinterpret_cast<f32x4*>(p.part_o + pr * D + d0) =
              f32x4{oacc[dt][nt][4 * jj] * inv, oacc[dt][nt][4 * jj + 1] * inv, oacc[dt][nt][4 * jj + 2] * inv,
                    oacc[dt][nt][4 * jj + 3] * inv};
        }
    }
    return;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l[nt] + swap_halves(l[nt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!valid[nt]) continue;
    if (h2 == 0) p.lse[orow[nt]] = lt > 0.f ? (m[nt] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d0 = 32 * dt + 8 * jj + 4 * h2;
        const float x0 = oacc[dt][nt][4 * jj] * inv, x1 = oacc[dt][nt][4 * jj + 1] * inv;
        const float x2 = oacc[dt][nt][4 * jj + 2] * inv, x3 = oacc[dt][nt][4 * jj + 3] * inv;
        if constexpr (OUT_BF16) {
          uint16_t* O = static_cast<uint16_t*>(p.o) + orow[nt] * D + d0;
          *reinterpret_cast<u32x2*>(O) =
              u32x2{static_cast<uint32_t>(f32_to_bf16_bits(x0)) | (static_cast<uint32_t>(f32_to_bf16_bits(x1)) << 16),
                    static_cast<uint32_t>(f32_to_bf16_bits(x2)) | (static_cast<uint32_t>(f32_to_bf16_bits(x3)) << 16)};
        } else {
          float* O = static_cast<float*>(p.o) + orow[nt] * D + d0;
          *reinterpret_cast<f32x4*>(O) = f32x4{x0, x1, x2, x3};
        }
      }
  }
}

// Merge of the split row groups' pieces.  One workgroup per (kv head, run of
// kMergeRowsPerLane * 256 / (d / 4) rows), looping over the split groups until the
// first unused entry; d / 4 lanes share a row, each lane takes kMergeRowsPerLane rows
// in one pass (rows merged in a loop would each pay a round of memory latency; 4 rows
// per lane measured slower than 1).  Per row: lse = M + ln sum_k exp(lse_k - M) with
// M the largest piece lse, and O = sum_k exp(lse_k - lse) O_k; a row no piece
// reaches gets O = 0, lse = -inf.  The grid is small and fixed, so a call that split
// nothing pays one short launch (a grid per possible split group was thousands of
// workgroups, each waiting for a compute unit the other stream's kernel held).
constexpr int kMergeRowsPerLane = 1;

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void fwd_merge_kernel(RowSplit sp, void* o, float* lse, int32_t n_blk, int32_t hq,
                                                        int32_t hkv) {
  constexpr int LPR = D / 4;                      // lanes per row, 4 values each
  constexpr int RPL = kMergeRowsPerLane;
  constexpr int RPW = 256 / LPR * RPL;            // rows per workgroup
  const int g = blockIdx.x % hkv;
  const int run = blockIdx.x / hkv;  // < kRowsPerGroup / RPW
  const int grp = hq / hkv;
  const int64_t R = static_cast<int64_t>(n_blk) * kBlock * grp;
  const int sub = threadIdx.x % LPR;
  int lr[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) lr[i] = run * RPW + i * (256 / LPR) + threadIdx.x / LPR;  // < kRowsPerGroup
  for (int sg = 0; sg < sp.max_pieces / 2; ++sg) {
    const int4 jb = sp.groups[sg];
    if (jb.x < 0) break;  // used entries come first
    auto prow = [&](int k, int i) { return (static_cast<int64_t>(jb.y + k) * hkv + g) * kRowsPerGroup + lr[i]; };
    // one pass over the pieces with a running maximum, so each piece's lse and O are
    // loaded together: den and acc are rescaled when the maximum grows
    float mx[RPL], den[RPL];
    f32x4 acc[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      mx[i] = -INFINITY;
      den[i] = 0.f;
      acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 2
    for (int k = 0; k < jb.z; ++k)
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const float lk = sp.part_lse[prow(k, i)];
        const f32x4 ok = *reinterpret_cast<const f32x4*>(sp.part_o + prow(k, i) * D + 4 * sub);
        if (lk == -INFINITY) continue;  // an empty piece adds nothing
        const float mnew = fmaxf(mx[i], lk);
        const float c = expf(mx[i] - mnew);  // 0 while mx is -inf
        const float wk = expf(lk - mnew);
        den[i] = den[i] * c + wk;
        acc[i] = acc[i] * c + wk * ok;
        mx[i] = mnew;
      }
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int64_t r = static_cast<int64_t>(jb.x) * kRowsPerGroup + lr[i];
      if (r >= R) continue;
      const f32x4 out = acc[i] * (den[i] > 0.f ? 1.f / den[i] : 0.f);
      const int64_t orow = (r / grp) * hq + static_cast<int64_t>(g) * grp + static_cast<int>(r % grp);
      if (sub == 0) lse[orow] = den[i] > 0.f ? mx[i] + logf(den[i]) : -INFINITY;
      if constexpr (OUT_BF16) {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(o) + orow * D + 4 * sub) = u32x2{
            static_cast<uint32_t>(f32_to_bf16_bits(out[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(out[1])) << 16),
            static_cast<uint32_t>(f32_to_bf16_bits(out[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(out[3])) << 16)};
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(o) + orow * D + 4 * sub) = out;
      }
    }
  }
}

#ifndef SXA_FWD_WAVES
#define SXA_FWD_WAVES 8
#endif
#ifndef SXA_FWD_STAGES
#define SXA_FWD_STAGES 3
#endif
#ifndef SXA_FWD_NT
#define SXA_FWD_NT 1
#endif
constexpr int kNT = SXA_FWD_NT;         // 32-row query tiles per wave
constexpr int kWaves = SXA_FWD_WAVES;   // waves sharing each K/V tile
constexpr int kStages = SXA_FWD_STAGES; // K/V tile buffers
constexpr int kRowsPerWG = 32 * kNT * kWaves;

template <int D, bool OUT_BF16>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.k_self = static_cast<const uint16_t*>(a.k_self);
  p.v_self = static_cast<const uint16_t*>(a.v_self);
  p.anchor = a.anchor;
  p.sample_start = a.sample_start;
  p.chunk_gstart = a.chunk_gstart;
  p.chunk_len = a.chunk_len;
  p.o = a.o;
  p.lse = a.lse;
  p.rg_order = a.rg_order;
  p.jobs = nullptr;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  p.n_blk = a.n_blk;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.n_chunk = a.n_chunk;
  p.scale_log2 = a.scale * kLog2e;
  const int64_t rows = static_cast<int64_t>(a.n_blk) * kBlock * (a.hq / a.hkv);
  const int64_t groups = (rows + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t n_wg = groups * a.hkv;
  if (n_wg == 0) return hipSuccess;
  if (a.row_split != nullptr && groups <= kMaxOrderedGroups && kRowsPerWG == kRowsPerGroup) {
    const RowSplit sp = row_split_layout(a.row_split, a);
    hipError_t e = launch_row_split_plan(a, sp, s);
    if (e != hipSuccess) return e;
    p.rg_order = nullptr;
    p.jobs = sp.jobs;
    p.part_o = sp.part_o;
    p.part_lse = sp.part_lse;
    fwd_bf16_kernel<D, kNT, kWaves, kStages, OUT_BF16>
        <<<dim3(static_cast<unsigned>((groups + sp.max_extra) * a.hkv)), dim3(64 * kWaves), 0, s>>>(p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int kRuns = kRowsPerGroup / (256 / (D / 4) * kMergeRowsPerLane);
    fwd_merge_kernel<D, OUT_BF16>
        <<<dim3(static_cast<unsigned>(a.hkv * kRuns)), dim3(256), 0, s>>>(sp, a.o, a.lse, a.n_blk, a.hq, a.hkv);
    return hipGetLastError();
  }
  if (p.rg_order != nullptr) {
    if (groups > kMaxOrderedGroups || kRowsPerWG != kRowsPerGroup) {
      p.rg_order = nullptr;
    } else {
      const hipError_t e = launch_row_group_order(a, kRowsPerWG, a.rg_order, s);
      if (e != hipSuccess) return e;
    }
  }
  fwd_bf16_kernel<D, kNT, kWaves, kStages, OUT_BF16>
      <<<dim3(static_cast<unsigned>(n_wg)), dim3(64 * kWaves), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.d == 64) return a.o_bf16 ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
  return a.o_bf16 ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace sxa
