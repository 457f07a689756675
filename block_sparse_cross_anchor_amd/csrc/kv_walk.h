// Key tiles visited by a query-major workgroup, and their copy into LDS.
//
// A workgroup owns consecutive query rows whose blocks span [b_first, b_last]; the
// keys any of them may read are its own blocks' rows (own-block term) and, in every
// local chunk, the positions in [min sample start, max anchor).  They are visited as
// 64-key tiles: own-block tiles first, then per chunk the tiles aligned to the chunk
// start that meet that interval.  Masking inside a tile is per row.
#pragma once
#include "device_common.h"
#include "lds_tile.h"

namespace sxa {

constexpr int kTileKeys = 64;

struct Tile {
  int64_t row0;  // first source row (local K/V row, or own-block row)
  int nrows;     // valid rows (<= 64)
  int coord0;    // key coordinate of row0: global position, or own-block row index
  int self;      // 1: own-block tile
};

// Position in the sequence of tiles of one workgroup (uniform across it).
struct Walk {
  int self_pos, self_end;
  int c;
  int64_t off;
  int gs, len, t, t_end;

  __device__ void start(bool with_self, int b_first, int b_last) {
    self_pos = with_self ? 16 * b_first : 0;
    self_end = with_self ? 16 * (b_last + 1) : 0;
    c = -1;
    off = 0;
    gs = len = t = t_end = 0;
  }
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
    // uniform index + constant address space: scalar loads, counted apart from
    // the vector-memory queue that the tile copies use
    const int c = __builtin_amdgcn_readfirstlane(w.c);
    w.gs = ((const __attribute__((address_space(4))) int32_t*)(cgs))[c];
    w.len = ((const __attribute__((address_space(4))) int32_t*)(clen))[c];
    const int a = max(LO, w.gs), e = min(HI, w.gs + w.len);
    if (a < e) {
      w.t = (a - w.gs) / kTileKeys;
      w.t_end = (e - w.gs + kTileKeys - 1) / kTileKeys;
    } else {
      w.t = w.t_end = 0;
    }
  }
}

// One 64-key tile (K rows, then V rows of one kv head) is copied straight from HBM
// into row-major swizzled LDS tiles with global_load_lds_dwordx4: lane i of a wave
// writes the 16 bytes at LDS offset 16 i of its 1 KiB slice, so each lane picks the
// global chunk that belongs at that position under the swizzle.  Rows past the tile
// end repeat its last row (those keys are masked; any finite value will do).  Every
// wave issues NI copies per tile.
template <int D, int WAVES>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int HALF = kTileKeys * CPR;  // chunks of K (or V) per tile
  static constexpr int NI = 2 * HALF / 64 / WAVES;
  static_assert(NI * 64 * WAVES == 2 * HALF, "tile must split evenly over the waves");
  static constexpr int ELEMS = 2 * kTileKeys * D;  // bf16 per buffer

  __device__ static __forceinline__ void issue(const Tile& t, const uint16_t* k, const uint16_t* v,
                                               const uint16_t* k_self, const uint16_t* v_self, int hkv,
                                               int g, int wave, int lane, uint16_t* buf) {
    const uint16_t* K = t.self ? k_self : k;
    const uint16_t* V = t.self ? v_self : v;
    const int last = t.nrows - 1;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int inst = wave * NI + j;
      const int c = inst * 64 + lane;
      const bool isv = c >= HALF;  // uniform per instruction
      const int cc = isv ? c - HALF : c;
      const int row = cc / CPR;
      const int logical = (cc % CPR) ^ LdsTile<D>::swz(row);
      const uint16_t* src = (isv ? V : K) + ((t.row0 + min(row, last)) * hkv + g) * D + 8 * logical;
      dma16(src, lds_addr(buf + inst * 512));
    }
  }
};

}  // namespace sxa
