// Device building blocks shared by the gfx950 attention kernels (forward and backward).
//
// MFMA: v_mfma_f32_32x32x16_bf16. For lane l (h32 = l / 32, l32 = l % 32) and element j:
//   A operand: A[l32][8 h32 + j]        B operand: B[8 h32 + j][l32]
//   accumulator element v: D[8 (v / 4) + 4 h32 + v % 4][l32]
//
// Two LDS layouts for a tile of 32 rows x 128 bf16 (8 KB), both filled by 16-byte
// global -> LDS copies (one 1 KB block of 4 rows per wave of an 8-wave workgroup):
//   row layout: chunk c (16 bytes) of row r sits at 16 (16 r + (c ^ swz(r))): a 32-row read
//     of one chunk (an MFMA A operand taken straight from rows) is free of bank conflicts;
//   transposed-read layout: 4-row blocks of 1 KB, each stored column-block first (the 16
//     chunks of one 32-dim block of the 4 rows are contiguous), read with
//     ds_read_b64_tr_b16 into an operand that holds a column of the tile; every such read
//     address is one lane base plus an immediate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsv_tiles {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) int lds_int;

constexpr int kRowBytes = 256;                 // 128 bf16
constexpr int kTileRows = 32;
constexpr int kTileBytes = kTileRows * kRowBytes;  // 8 KB

// 16-byte chunk swizzle of a row in the row layout: chunk c of row r lives at chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Nothing may be scheduled across this point (keeps a hand-placed MFMA / VALU interleave).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// max / sum with the partner lane l ^ 32.
__device__ __forceinline__ float pair_max(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N of this wave's memory loads are outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte global -> LDS copy per lane from base + voff: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16). Issued from inline asm so that the compiler does not add
// its own conservative waits on LDS reads; every wait on these copies is explicit
// (wait_vmcnt) and so is the barrier. M0 (the LDS destination base) is written only by
// these copies in these kernels, so the clobber of the reserved register is safe; the
// compiler's note about it is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(unsigned voff, const char* base, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(lds_wave_base), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that waits for this wave's LDS reads but not for its prefetches.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Copy lane of the row layout: lane i of wave w copies row 4w + i / 16, and its 16 bytes
// land in chunk (i % 16) ^ swz(row) of that row; returns the row and the byte offset of
// the source chunk inside the row.
__device__ __forceinline__ void row_copy_lane(int wave, int i, int& row, unsigned& off) {
  row = 4 * wave + (i >> 4);
  off = (unsigned)(((i & 15) ^ swz(row)) * 16);
}

// Copy lane of the transposed-read layout: lane i of wave w copies row 4w + (i / 4) % 4,
// chunk 4 (i / 16) + i % 4.
__device__ __forceinline__ void tr_copy_lane(int wave, int i, int& row, unsigned& off) {
  row = 4 * wave + ((i >> 2) & 3);
  off = (unsigned)((4 * (i >> 4) + (i & 3)) * 16);
}

// Row-layout read address of row l32, 16-column step s (columns 16 s + 8 h32 .. +7): the
// MFMA A operand A[l32][8 h32 + j] of a tile whose rows are the A rows.
__device__ __forceinline__ unsigned row_read_addr(unsigned tile, int l32, int h32, int s) {
  return tile + l32 * kRowBytes + ((((2 * s) | h32) ^ swz(l32)) << 4);
}

__device__ __forceinline__ bf16x8 lds_row(unsigned addr) { return *(lds_bf16x8*)(uintptr_t)addr; }

// Transposed-read lane base: lane i of 16-lane group (h32, g2) reads 8 bytes of row
// 16 kc + 8 rd + 4 h32 + i / 4, columns 32 db + 16 g2 + 4 (i % 4) .. +3, i.e. chunk
// 4 db + 2 g2 + (i % 4) / 2 of 4-row block 4 kc + 2 rd + h32 (kc: row chunk of 16, rd:
// its half, db: 32-column block).
__device__ __forceinline__ unsigned tr_read_base(unsigned tile, int lane) {
  const int i = lane & 15, g2 = (lane >> 4) & 1, h32 = lane >> 5;
  return tile + 1024 * h32 + 16 * (4 * (i >> 2) + 2 * g2 + ((i & 3) >> 1)) + 8 * (i & 1);
}

__device__ __forceinline__ bf16x8 lds_tr(unsigned a0, unsigned a1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
  u32x4 u;
  u[0] = __builtin_bit_cast(u32x2, a)[0];
  u[1] = __builtin_bit_cast(u32x2, a)[1];
  u[2] = __builtin_bit_cast(u32x2, b)[0];
  u[3] = __builtin_bit_cast(u32x2, b)[1];
  return __builtin_bit_cast(bf16x8, u);
}

// Transposed operand i (row chunk kc = i / 4, column block db = i % 4) of the tile at byte
// offset `slot` from the lane base: the MFMA A operand A[m][k] = tile[row(k)][32 db + m],
// where the reduction index k = 8 h + j of 16-row chunk kc maps to the tile row
// 16 kc + 8 (j / 4) + 4 h + j % 4 -- the row that an accumulator's element 8 kc + j holds
// in lane half h (so an accumulator converted to bf16 is the matching B operand as is).
__device__ __forceinline__ bf16x8 tr_operand(unsigned base, unsigned slot, int i) {
  const int kc = i >> 2, db = i & 3;
  const unsigned a = base + slot + 4096 * kc + 256 * db;
  return lds_tr(a, a + 2048);
}

}  // namespace lsv_tiles
