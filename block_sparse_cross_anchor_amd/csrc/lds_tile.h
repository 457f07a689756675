// Row-major bf16 tiles in LDS and the two ways the MFMA kernels read them.
//
// A tile holds rows of D bf16 values (D / 8 chunks of 16 bytes).  The chunk index
// is XOR-ed with a function of the row (swz) chosen so that both read patterns
// below are free of LDS bank conflicts (checked with SQ_LDS_BANK_CONFLICT).
//
//  * frag(): one 16-byte read per lane -- row `row`, 8 consecutive columns
//    starting at 8 * chunk.  Used for MFMA operands whose contraction index runs
//    along the row (e.g. K or Q with the head dimension contracted).
//  * frag_t(): the transposed operand.  gfx950's ds_read_b64_tr_b16 reads 8 bytes
//    per lane and, inside each group of 16 lanes, hands output lane 4c + e the
//    e-th 16-bit element of the reads of lanes c, c + 4, c + 8 and c + 12.  If lane
//    s of the group points at row rows[s / 4], columns col + 4 * (s % 4) .. + 3,
//    output lane i receives column col + i of rows rows[0..3].  Two such reads
//    give a lane 8 rows of one column: the MFMA operand of X^T whose contraction
//    index runs over rows (V^T for P V, K^T for dS K, Q^T / dO^T for dK / dV).
#pragma once
#include "device_common.h"

namespace sxa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct LdsTile {
  static constexpr int CPR = D / 8;  // 16-byte chunks per row

  // Chunk swizzle f(row): a bijection on the low row bits, so 16 lanes reading 16
  // consecutive rows at one chunk hit 16 distinct chunk positions; and the 4
  // consecutive rows of one transposing read land in 4 different groups of 4
  // chunks, so its 4 rows x 4 chunks (32 lanes) cover every bank once.
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);  // 128-byte rows: two per bank sweep
  }
  __device__ static __forceinline__ int phys(int row, int chunk) { return chunk ^ swz(row); }

  __device__ static __forceinline__ void store(uint16_t* t, int row, int chunk, const u32x4& v) {
    *reinterpret_cast<u32x4*>(t + row * D + 8 * phys(row, chunk)) = v;
  }

  __device__ static __forceinline__ bf16x8 frag(const uint16_t* t, int row, int chunk) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t + row * D + 8 * phys(row, chunk)));
  }

  // lane s (0..15) of its 16-lane group: rows r4[s / 4] of the first read and
  // r4b[s / 4] of the second; columns col + 4 * (s % 4).  `col` is a multiple of 16.
  __device__ static __forceinline__ bf16x8 frag_t(const uint16_t* t, int row_a, int row_b, int col, int s) {
    const int c = col + 4 * (s & 3);
    const int chunk = c >> 3, within = c & 7;
    const uint16_t* pa = t + row_a * D + 8 * phys(row_a, chunk) + within;
    const uint16_t* pb = t + row_b * D + 8 * phys(row_b, chunk) + within;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pb));
    // combine through 32-bit words (element-wise __bf16 bit casts are not reliable)
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
  }

  // Offset form for loops over k-steps, on tiles whose base is 256-byte aligned.  A
  // row is 2 D bytes and the swizzle only permutes the 16-byte chunk bits inside it,
  // so the step-dependent part of an address is a constant XOR:
  //   frag(row, 2 ks + h)        at byte  frag_off(row, h) ^ (32 ks)
  //   frag_t(rows of k-step kq, col = 32 dt + 16 hb)
  //                              at bytes tr_off(r, hb, s) ^ (64 dt) + kq 16 rows,
  //                              r = 4 h + s / 4 (first read) or 8 + 4 h + s / 4.
  __device__ static __forceinline__ int frag_off(int row, int h) { return row * 2 * D + 16 * (h ^ swz(row)); }
  __device__ static __forceinline__ int tr_off(int row, int hb, int s) {
    const int lowc = 2 * hb + ((s & 3) >> 1);  // chunk bits below the column-block bits
    return row * 2 * D + 16 * (lowc ^ swz(row)) + 8 * (s & 1);
  }
  __device__ static __forceinline__ bf16x8 frag_at(const uint16_t* base, int byte_off) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + byte_off));
  }
  __device__ static __forceinline__ bf16x8 frag_t_at(const uint16_t* base, int off_a, int off_b) {
    const char* b8 = reinterpret_cast<const char*>(base);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b8 + off_a));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b8 + off_b));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
  }
};

// Reads at raw LDS byte addresses (32-bit, as lds_addr() gives them), for loops that
// keep one per-lane base address and vary it by XOR / immediate offsets.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ bf16x8 lds_frag(uint32_t addr) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<lds_u32x4*>(addr));
}
__device__ __forceinline__ bf16x8 lds_frag_t(uint32_t addr_a, uint32_t addr_b) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(addr_a));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4*>(addr_b));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
}

// Key order shared by P (or dS) held in MFMA accumulator registers and the
// transposed operand that multiplies it: in k-step ks (16 keys) lane half h holds,
// at positions i = 0..7, the keys 16 ks + 8 (i / 4) + 4 h + i % 4.  frag_t reads
// positions 0..3 from rows 16 ks + 4 h + (s / 4) and 4..7 from 16 ks + 8 + 4 h + (s / 4).
__device__ __forceinline__ int tr_row_a(int ks, int h, int s) { return 16 * ks + 4 * h + (s >> 2); }
__device__ __forceinline__ int tr_row_b(int ks, int h, int s) { return 16 * ks + 8 + 4 * h + (s >> 2); }

// 16-byte direct HBM -> LDS copy (global_load_lds_dwordx4): lane i of the wave
// writes LDS bytes [lds_base + 16 i, +16).  Issued from asm so that the compiler
// does not add its own conservative waits for it; the caller waits with
// wait_vmcnt<>() and a bare s_barrier before any wave reads the destination.
// The instruction writes no VGPR, so nothing in flight can clobber a register.
// m0 (which the compiler reserves) is saved and restored around it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);  // wave-uniform by contract
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(base)
      : "memory");
}

// 4-byte variant (global_load_lds_dword): lane i writes LDS bytes [lds_base + 4 i, +4).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(base)
      : "memory");
}

// Scalar-base forms: the wave-uniform 64-bit base sits in SGPRs and each lane adds a
// 32-bit byte offset (one VGPR per copy instead of a 64-bit address).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(uniform_ptr(sbase)), "s"(base)
      : "memory");
}

// Two or four 16-byte copies from one uniform base, to LDS slices lds_base +
// 1024 j, in one block: m0 is saved and restored once.  An s_nop follows each m0
// write ahead of the copy that reads it.
__device__ __forceinline__ void dma16_s2(const void* sbase, uint32_t o0, uint32_t o1, uint32_t lds_base) {
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_base), b1 = b0 + 1024;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "s"(uniform_ptr(sbase)), "s"(b0), "s"(b1)
      : "memory");
}

__device__ __forceinline__ void dma16_s4(const void* sbase, uint32_t o0, uint32_t o1, uint32_t o2, uint32_t o3,
                                         uint32_t lds_base) {
  const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_base);
  const uint32_t b1 = b0 + 1024, b2 = b0 + 2048, b3 = b0 + 3072;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %5\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %5\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(uniform_ptr(sbase)), "s"(b0), "s"(b1), "s"(b2), "s"(b3)
      : "memory");
}

__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(uniform_ptr(sbase)), "s"(base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
}

// Wait until at most VM vector-memory operations of this wave are outstanding.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that publishes this wave's LDS writes (lgkmcnt(0)) but does not
// wait for vector-memory operations, so copies and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier without a memory fence (the fence of __syncthreads would also
// wait for every DMA still in flight).  LDS written by ds_write must be waited for
// (lgkmcnt) by the writer before it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace sxa
