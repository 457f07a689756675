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

// Position in the sequence of tiles of one workgroup (uniform across it).  The
// own-block rows form the first run of tiles, then each chunk that meets the
// interval.  The next tile of the current run is held ready (source row, key
// coordinate, tiles left in the run, rows from it to the run's end), so a step is a
// handful of scalar operations with no branch; only a change of run branches.
// Once exhausted, walk_next keeps returning false.
struct Walk {
  int nc;         // next chunk to examine
  int64_t off;    // local row of chunk nc
  int64_t row;    // next tile: source row
  int coord;      //            key coordinate
  int left;       //            tiles left in its run, itself included
  int rows_left;  //            rows from it to its run's end
  int self;       //            1: own-block run

  __device__ void start(bool with_self, int b_first, int b_last) {
    nc = 0;
    off = 0;
    row = with_self ? 16 * b_first : 0;
    coord = static_cast<int>(row);
    rows_left = with_self ? 16 * (b_last - b_first + 1) : 0;
    left = (rows_left + kTileKeys - 1) / kTileKeys;
    self = 1;
  }
};

__device__ __forceinline__ bool walk_next(Walk& w, const int32_t* __restrict__ cgs,
                                          const int32_t* __restrict__ clen, int n_chunk, int LO,
                                          int HI, Tile& out) {
  if (__builtin_expect(w.left == 0, 0)) {  // next chunk that meets [LO, HI)
    while (true) {
      if (w.nc >= n_chunk) return false;
      // uniform index + constant address space: scalar loads, counted apart from
      // the vector-memory queue that the tile copies use
      const int c = __builtin_amdgcn_readfirstlane(w.nc);
      const int gs = ((const __attribute__((address_space(4))) int32_t*)(cgs))[c];
      const int len = ((const __attribute__((address_space(4))) int32_t*)(clen))[c];
      const int64_t off = w.off;
      w.off += len;
      ++w.nc;
      const int a = max(LO, gs), e = min(HI, gs + len);
      if (a < e) {
        const int t = (a - gs) / kTileKeys;
        w.row = off + static_cast<int64_t>(t) * kTileKeys;
        w.coord = gs + t * kTileKeys;
        w.left = (e - gs + kTileKeys - 1) / kTileKeys - t;
        w.rows_left = len - t * kTileKeys;
        w.self = 0;
        break;
      }
    }
  }
  out.row0 = w.row;
  out.nrows = min(kTileKeys, w.rows_left);
  out.coord0 = w.coord;
  out.self = w.self;
  w.row += kTileKeys;
  w.coord += kTileKeys;
  w.rows_left -= kTileKeys;
  --w.left;
  return true;
}

// One 64-key tile (K rows, then V rows of one kv head) is copied straight from HBM
// into row-major swizzled LDS tiles with global_load_lds_dwordx4: lane i of a wave
// writes the 16 bytes at LDS offset 16 i of its 1 KiB slice, so each lane picks the
// global chunk that belongs at that position under the swizzle.  Rows past the tile
// end repeat its last row (those keys are masked; any finite value will do).  Every
// wave issues NI copies per tile.  The address is the tile's first element (uniform,
// in scalar registers) plus a 32-bit per-lane byte offset.  With KEEP the offsets
// of a full tile (the same for every tile) are computed once and held in registers;
// without, they are recomputed per tile (a kernel with no registers to spare).
template <int D, int WAVES, bool KEEP>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int HALF = kTileKeys * CPR;  // chunks of K (or V) per tile
  static constexpr int NI = 2 * HALF / 64 / WAVES;
  static_assert(NI * 64 * WAVES == 2 * HALF, "tile must split evenly over the waves");
  static_assert(HALF % 64 == 0, "an instruction copies K or V, never both");
  static constexpr int ELEMS = 2 * kTileKeys * D;  // bf16 per buffer

  int w;            // wave index (uniform)
  uint32_t stride;  // bytes per source row: hkv * D * 2 (< 2^24, so 24-bit products suffice)
  uint32_t voff[KEEP ? NI : 1];

  // chunk `cc` of K or V: its row in the tile and the byte offset of its 16 bytes
  // inside that row under the swizzle
  __device__ static __forceinline__ uint32_t row_of(uint32_t cc) { return cc / CPR; }
  __device__ static __forceinline__ uint32_t col_bytes(uint32_t cc) {
    return 16 * ((cc % CPR) ^ LdsTile<D>::swz(static_cast<int>(cc / CPR)));
  }
  __device__ static __forceinline__ uint32_t chunk(int inst, int lane) {
    return static_cast<uint32_t>(inst * 64 - (inst * 64 >= HALF ? HALF : 0) + lane);
  }

  __device__ __forceinline__ TileDma(int hkv, int wave, int lane) {
    w = __builtin_amdgcn_readfirstlane(wave);
    stride = static_cast<uint32_t>(hkv) * D * 2;
#pragma unroll
    for (int j = 0; j < (KEEP ? NI : 1); ++j) {
      const uint32_t cc = chunk(w * NI + j, lane);
      voff[j] = __umul24(row_of(cc), stride) + col_bytes(cc);
    }
  }

  // lds: byte address of the tile buffer in LDS
  __device__ __forceinline__ void issue(const Tile& t, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* k_self, const uint16_t* v_self, int hkv, int g,
                                        int lane, uint32_t lds) const {
    const uint16_t* K = t.self ? k_self : k;
    const uint16_t* V = t.self ? v_self : v;
    const int64_t first = (t.row0 * hkv + g) * D;  // element offset of the tile's row 0
    const uint32_t lb = lds + static_cast<uint32_t>(w * NI * 1024);
    if (KEEP && t.nrows == kTileKeys) {
      if constexpr (NI == 4 || NI == 2) {  // a wave's copies all come from K, or all from V
        static_assert(HALF % (NI * 64) == 0, "a wave's copies stay inside K or inside V");
        const uint16_t* src = (w * NI * 64 >= HALF ? V : K) + first;
        if constexpr (NI == 4) dma16_s4(src, voff[0], voff[KEEP ? 1 : 0], voff[KEEP ? 2 : 0], voff[KEEP ? 3 : 0], lb);
        else dma16_s2(src, voff[0], voff[KEEP ? 1 : 0], lb);
      } else {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const bool isv = (w * NI + j) * 64 >= HALF;  // uniform per instruction
          dma16_s((isv ? V : K) + first, voff[KEEP ? j : 0], lb + 1024 * j);
        }
      }
    } else {
      const uint32_t last = static_cast<uint32_t>(t.nrows - 1);
      int ln = lane;
      asm volatile("" : "+v"(ln));  // recomputed here, not hoisted into held registers
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const bool isv = (w * NI + j) * 64 >= HALF;
        const uint32_t cc = chunk(w * NI + j, ln);
        const uint32_t o = __umul24(min(row_of(cc), last), stride) + col_bytes(cc);
        dma16_s((isv ? V : K) + first, o, lb + 1024 * j);
      }
    }
  }
};

}  // namespace sxa
