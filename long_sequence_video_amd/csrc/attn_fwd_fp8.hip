// FP8 (e4m3) variant of the dense non-causal varlen attention forward for gfx950 (MI355X).
//
// The operation: TensorRT-LLM PR #21275 (the MiniMax-H3 recipe commit: cuDNN attention with
// --qk-dtype fp8 --v-dtype fp8, per-tensor FP8 descales, the LSE returned) over the varlen
// forward of FastVideo #2049 (flash_attn_cute.py). Inputs are OCP e4m3 bytes with per-tensor
// descales dq, dk, dv; for every segment, head and query row i:
//   z_ij = scale dq dk (q8_i . k8_j),  O_i = dv sum_j softmax_j(z_ij) v8_j,  LSE_i = ln sum_j e^z_ij.
//
// Design (gfx950, wave64), following the BF16 kernel:
//  * One workgroup = 8 waves = 256 query rows, two waves per SIMD; each wave owns 32 queries.
//  * Key tiles of 64 rows (one v_mfma_f32_32x32x64_f8f6f4 reduces over 64): S^T = K Q^T is four
//    MFMAs per tile (two 32-key halves x two 64-dim halves), A = K rows from LDS, B = Q^T in
//    registers; a lane gets one query and 32 of the 64 keys (16 per half).
//  * P is quantised to e4m3 in place of the score accumulators and is the B operand of
//    O^T += V^T P^T (four MFMAs, one per 32-dim block): the MFMA pairs byte j of an A lane
//    with byte j of the B lane of the same half, so P's bytes only need V^T's bytes in the
//    same key order; V^T is read with ds_read_b64_tr_b8 (a lane gets one column of 8 rows).
//  * The sum of the quantised weights comes from one more, half-size MFMA per tile
//    (v_mfma_f32_16x16x128_f8f6f4 with a 0/1 selection A that routes each query's 64 bytes
//    of P into one output element): O is divided by exactly the weights its product used
//    (no fp8 dot instruction on gfx950). The LSE uses the fp32 sum of the unquantised weights.
//  * Software pipeline per key tile t: one sequence of nine MFMAs, S(t+1) = Q K(t+1)^T, then
//    O += P(t-1) V(t-1) and the weight sum of P(t-1), with the exp2 / e4m3 work of S(t) placed
//    between them (scheduling barriers hold the order). The running max is checked after the
//    tile, and only when this lane's weights of the tile sum past what a raise requires.
//  * Softmax: p = exp2(s c - m c + 5) with c = scale dq dk log2(e) and m a running row max
//    raised only when a tile exceeds it by more than 3 log2 units (then O and the sums are
//    rescaled, O after the tile's MFMAs): weights stay in [0, 2^8], below e4m3's 448 (its
//    conversion does not saturate), and keys up to ~14 log2 units below the max keep a
//    representable weight. A fixed
//    first-tile reference, as in the BF16 kernel, would overflow e4m3's range whenever a
//    later key exceeds the first tile by 3.8 log2 units, which long rows do routinely.
//  * LDS: K and V rows of 128 bytes with 16-byte chunk c of row r stored at c ^ sw8(r), a
//    permutation of the row-pair index that keeps the row reads and the transposed reads free
//    of bank conflicts. K and V stream through an 8-slot ring, 5 tiles ahead, one barrier per two
//    tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "lsv.h"
#include "tile_ops.h"

namespace {

using namespace lsv_tiles;

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBQ = kWaves * 32;          // query rows per workgroup
constexpr int kBK = 64;                   // keys per tile
constexpr int kRow8 = kD;                 // bytes per fp8 row
constexpr int kSlot = kBK * kRow8;        // 8 KB per tile
constexpr int kSlots = 8;
constexpr int kAhead = 5;
constexpr int kRingBytes = kSlots * kSlot;
constexpr int kLdsBytes = 2 * kRingBytes;
constexpr int kOpsPerTile = 2;            // one 1 KB copy of K and one of V per wave per tile
constexpr float kRefLog2 = 5.0f;          // the reference weight: 2^5
constexpr float kLazyLog2 = 3.0f;         // raise the running max only beyond this (log2 units)
// A weight above 2^(kRefLog2 + kLazyLog2) = 256 puts its lane's tile sum above this (a sum of
// non-negative terms is at least its largest term, up to fp32 rounding of ~2^-19 relative).
constexpr float kCheckSum = 255.0f;
static_assert(kRefLog2 + kLazyLog2 == 8.0f, "kCheckSum assumes a raise threshold of 2^8");
constexpr unsigned kOnes = 0x38383838u;   // four e4m3 ones
// The workgroup synchronises after odd tiles only. Between two barriers a wave runs at most
// tiles t+1, t+2 (t odd) and copies tiles t+1+kAhead, t+2+kAhead; a wave still behind has
// finished tile t, so it may read V(t), K(t+2) (tile t+1) or V(t+1), K(t+3) (tile t+2): the
// written slots must be none of tiles t .. t+3, i.e. kAhead <= kSlots - 3. Each barrier
// follows the wait for tile t+3 (read as K by tile t+2), leaving kAhead - 3 tiles in flight.
static_assert(kAhead >= 3 && kAhead <= kSlots - 3, "ring too small for the prefetch distance");

// Chunk swizzle of a row: with k = (row / 2) % 8 (rows 2k and 2k + 1 sit in the two halves of
// the 64 banks), 4 (k % 2) + k / 2. Any 8 even (or odd) rows of a 16-row block get 8 distinct
// values (row reads), and the row pairs of one transposed read, k in {0, 1, 4, 5} or
// {2, 3, 6, 7}, get distinct value / 2, so the two 16-lane groups of a 32-lane half, which
// read adjacent chunks of the same rows, meet no bank twice. A function of k only: rows 32 and
// 16 apart share it (immediate read offsets).
__device__ __forceinline__ int sw8(int row) {
  const int k = (row >> 1) & 7;
  return ((k & 1) << 2) | (k >> 1);
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Key of byte j (0..31) of a P^T / V^T operand in lane half h: byte j = 16 a + v holds
// accumulator element v of key half a, i.e. key 32 a + 8 (v / 4) + 4 h + v % 4.
__device__ __forceinline__ int key_of(int h, int j) {
  return 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h + (j & 3);
}

struct Lane {
  int lane, h32, l32;
  unsigned kaddr[4];   // K row reads, ring slot 0, key half 0: index 2 c2 + sub (key half a: + 4096 a)
  unsigned vaddr[4];   // V^T transposed reads, V ring slot 0, read 0: index db (read r: + 2048 r)
};

struct Ctx {
  unsigned lds_copy;   // this wave's 1 KB block of ring slot 0 (uniform)
  const char* kbase;   // k row seg_start, this head (uniform)
  const char* vbase;
  unsigned row_stride;
  int crow;            // the tile row this lane copies
  unsigned coff;       // the byte offset of its chunk inside the row
  unsigned cconst;     // crow * row_stride + coff
  int seg_len;
  float c;             // scale dq dk log2(e)
  float lazy;          // kLazyLog2 / c: the max margin in raw score units
};

struct Acc {
  f32x16 O[4];   // O^T, d-block db
  f32x4 LB;      // element 0 of lanes 0..31: sum of the quantised weights of query l32 (else 0)
  float m;       // running row max (raw score units)
  float l;       // fp32 sum of the weights, for the LSE
};

// Tile t (segments of 64 keys or more): rows min(64 t, seg_len - 64) .. +63; wave w copies
// rows 8w .. 8w+7, lane i the 16 bytes of LDS chunk position i % 8 of row 8w + i / 8.
__device__ __forceinline__ void load_tile(const Ctx& cx, int t) {
  const unsigned slot = (unsigned)(t & (kSlots - 1)) * kSlot;
  const unsigned off = (unsigned)min(t * kBK, cx.seg_len - kBK) * cx.row_stride;
  dma16(cx.cconst, cx.kbase + off, cx.lds_copy + slot);
  dma16(cx.cconst, cx.vbase + off, cx.lds_copy + slot + kRingBytes);
}
// A single tile shorter than 64 keys: rows past the segment repeat its last row.
__device__ __forceinline__ void load_tile_short(const Ctx& cx, int t) {
  const unsigned slot = (unsigned)(t & (kSlots - 1)) * kSlot;
  const unsigned r = (unsigned)min(cx.crow, cx.seg_len - 1);
  dma16(__umul24(r, cx.row_stride) + cx.coff, cx.kbase, cx.lds_copy + slot);
  dma16(__umul24(r, cx.row_stride) + cx.coff, cx.vbase, cx.lds_copy + slot + kRingBytes);
}

// Lane read bases of one ring slot (one add each; the rest of every read address is an
// immediate offset).
struct Bases {
  unsigned k[4], v[4];
};
__device__ __forceinline__ Bases bases(const Lane& ln, unsigned kslot, unsigned vslot) {
  Bases b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b.k[i] = ln.kaddr[i] + kslot;
    b.v[i] = ln.vaddr[i] + vslot;
  }
  return b;
}

__device__ __forceinline__ i32x8 k_operand(const Bases& b, int a, int c2) {
  const u32x4 x = *(lds_u32x4*)(uintptr_t)(b.k[2 * c2] + 4096u * a);
  const u32x4 y = *(lds_u32x4*)(uintptr_t)(b.k[2 * c2 + 1] + 4096u * a);
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (int)x[i];
    r[4 + i] = (int)y[i];
  }
  return r;
}

__device__ __forceinline__ i32x8 v_operand(const Bases& b, int db) {
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)(b.v[db] + 2048u * q));
    r[2 * q] = x[0];
    r[2 * q + 1] = x[1];
  }
  return r;
}

// S^T for the two key halves of a tile.
__device__ __forceinline__ void qk_tile(const Bases& b, const i32x8 (&qr)[2], f32x16 (&S)[2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    f32x16 s = {};
    s = mfma8(k_operand(b, a, 0), qr[0], s);
    s = mfma8(k_operand(b, a, 1), qr[1], s);
    S[a] = s;
  }
}

// Keys of the tile before `skip` (shifted last tile) or from `valid` on (short tile) get -inf.
__device__ __forceinline__ void mask_head(f32x16 (&S)[2], int skip, int h32) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (32 * a + 8 * (v >> 2) + 4 * h32 + (v & 3) < skip) S[a][v] = -INFINITY;
}
__device__ __forceinline__ void mask_tail(f32x16 (&S)[2], int valid, int h32) {
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (32 * a + 8 * (v >> 2) + 4 * h32 + (v & 3) >= valid) S[a][v] = -INFINITY;
}

// Max over the row (this lane's 32 scores and its partner's).
__device__ __forceinline__ float row_max(const f32x16 (&S)[2]) {
  float m = fmaxf(S[0][0], S[1][0]);
#pragma unroll
  for (int v = 1; v < 16; ++v) m = fmaxf(fmaxf(m, S[0][v]), S[1][v]);
  return pair_max(m);
}

// Weights of 4 consecutive bytes (dword w of the P operand): exp2(s c + nr), summed into l,
// quantised to e4m3. The upper half of P[w] is written by the second conversion, so the
// first one may keep whatever P[w] held.
__device__ __forceinline__ void softmax_dword(const f32x16 (&S)[2], i32x8& P, float& l, float c, float nr, int w) {
  const int a = w >> 2, v0 = 4 * (w & 3);
  float e[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    e[b] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[a][v0 + b], c, nr));
    l += e[b];
  }
  unsigned d = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], (unsigned)P[w], false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], d, true);
  P[w] = (int)d;
}
__device__ __forceinline__ void softmax_all(const f32x16 (&S)[2], i32x8& P, float& l, float c, float nr) {
#pragma unroll
  for (int w = 0; w < 8; ++w) softmax_dword(S, P, l, c, nr, w);
}

// The weight sums: one 16x16x128 MFMA whose A selects, for output row 0, the lanes of
// queries 0..15 (lane blocks 0 and 2 of B) and, for row 4, those of queries 16..31 (blocks 1
// and 3); row 0 lands in element 0 of lanes 0..15 and row 4 in element 0 of lanes 16..31,
// i.e. each sum in the lane whose l32 is its query.
__device__ __forceinline__ f32x4 mfma_sum(const i32x8& sel, const i32x8& P, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, P, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void pv_tile(Acc& acc, const Bases& b, const i32x8& P, const i32x8& sel) {
#pragma unroll
  for (int db = 0; db < 4; ++db) acc.O[db] = mfma8(v_operand(b, db), P, acc.O[db]);
  acc.LB = mfma_sum(sel, P, acc.LB);
}

// Raising the running max from m to mnew rescales everything summed against m by
// r = exp2((m - mnew) c).
__device__ __forceinline__ void scale_o(Acc& acc, float r) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc.O[db][v] *= r;
  acc.LB[0] *= r;
}

__device__ __forceinline__ unsigned slot_of(int t) { return (unsigned)(t & (kSlots - 1)) * kSlot; }

// LDS operands are read this many MFMAs ahead of their use (1 and 3 measured slower).
constexpr int kReadAhead = 2;

// Steady-state key tile t (1 <= t <= n_kt - 2). On entry S(t) and P(t-1) are complete and
// tile t+1 is in LDS. One sequence of nine MFMAs, S(t+1) = Q K(t+1)^T (four, first), O +=
// P(t-1) V(t-1) (four) and the weight sum of P(t-1), with the weights P(t) of S(t), against the
// running max, computed between them, operands read two MFMAs ahead and the copy of tile
// t + kAhead issued after the fifth. Then the lazy max check of S(t), gated so that the row max
// is computed only when a raise is possible (rare); a raise rescales l, O and the weight sums
// and redoes P(t). After an odd tile, tile t+3 is waited for and the workgroup synchronises.
template <int U>
__device__ __forceinline__ void step(const Ctx& cx, int t, Acc& acc, const f32x16 (&Scur)[2], f32x16 (&Snext)[2],
                                     const i32x8& Pprev, i32x8& Pcur, const i32x8 (&qr)[2], const Lane& ln,
                                     const i32x8& sel) {
  const float nr = kRefLog2 - acc.m * cx.c;
  // t % kSlots == U: both ring slots are compile-time offsets (LDS read immediates).
  const Bases b = bases(ln, ((U + 1) % kSlots) * kSlot, ((U + kSlots - 1) % kSlots) * kSlot);
  i32x8 opnd[9];
  auto read = [&](int n) {
    if (n < 4) opnd[n] = k_operand(b, n >> 1, n & 1);
    else if (n < 8) opnd[n] = v_operand(b, n - 4);
  };
#pragma unroll
  for (int n = 0; n < kReadAhead; ++n) read(n);
  sched_fence();
  f32x16 s = {};
  float ls = 0.f;  // this tile's weights, this lane's 32 keys
#pragma unroll
  for (int n = 0; n < 9; ++n) {
    if (n < 4) {
      const int a = n >> 1, c2 = n & 1;
      s = mfma8(opnd[n], qr[c2], c2 ? s : f32x16{});
      if (c2) Snext[a] = s;
    } else if (n < 8) {
      acc.O[n - 4] = mfma8(opnd[n], Pprev, acc.O[n - 4]);
    } else {
      acc.LB = mfma_sum(sel, Pprev, acc.LB);
    }
    if (n + kReadAhead < 9) read(n + kReadAhead);
    if (n == 4) load_tile(cx, t + kAhead);
    if (n < 8) softmax_dword(Scur, Pcur, ls, cx.c, nr, n);
    sched_fence();
  }
  // P(t) and its sum must be complete here (they must not sink into the next tile).
  asm volatile("" : "+v"(Pcur), "+v"(ls));
  // The lazy max check, gated: a raise needs a score above m + lazy, i.e. a weight above
  // 2^(kRefLog2 + kLazyLog2), and so this lane's tile sum above kCheckSum. Only then (rare) is
  // the row max computed; on a raise, l, O and the weight sums are rescaled (O after this
  // tile's MFMAs, which still add P(t-1) weighted against the old max) and P(t) is redone.
  if (__builtin_amdgcn_ballot_w64(ls > kCheckSum) != 0) {
    const float mx = row_max(Scur);
    if (__builtin_amdgcn_ballot_w64(mx > acc.m + cx.lazy) != 0) {  // wave-uniform
      const float mnew = fmaxf(acc.m, mx);
      const float r = __builtin_amdgcn_exp2f((acc.m - mnew) * cx.c);
      acc.l *= r;
      acc.m = mnew;
      ls = 0.f;
      softmax_all(Scur, Pcur, ls, cx.c, kRefLog2 - mnew * cx.c);
      scale_o(acc, r);
    }
  }
  acc.l += ls;
  if (U & 1) {
    wait_vmcnt<kOpsPerTile * (kAhead - 3)>();
    barrier_lds();
  }
}

// The last tile tl = n_kt - 1 >= 1 (loaded shifted to end at the segment end): P(tl-1) V(tl-1),
// the masked scores S(tl), the max check, P(tl) V(tl).
__device__ __forceinline__ void last_tile(const Ctx& cx, int n_kt, Acc& acc, f32x16 (&Slast)[2], const i32x8& Pprev,
                                          i32x8& Pcur, const Lane& ln, const i32x8& sel) {
  const int tl = n_kt - 1;
  pv_tile(acc, bases(ln, 0, slot_of(tl - 1)), Pprev, sel);
  mask_head(Slast, kBK * n_kt - cx.seg_len, ln.h32);
  const float mx = row_max(Slast);
  if (__builtin_amdgcn_ballot_w64(mx > acc.m + cx.lazy) != 0) {
    const float mnew = fmaxf(acc.m, mx);
    const float r = __builtin_amdgcn_exp2f((acc.m - mnew) * cx.c);
    acc.l *= r;
    acc.m = mnew;
    scale_o(acc, r);
  }
  softmax_all(Slast, Pcur, acc.l, cx.c, kRefLog2 - acc.m * cx.c);
  pv_tile(acc, bases(ln, 0, slot_of(tl)), Pcur, sel);
}

// The key loop: online softmax with a lazily raised row max. The first tile sets the max;
// later a tile raises it (and O and the sums are rescaled) only when some row of the wave
// exceeds it by more than 3 log2 units, which is wave-uniform and rare after the first tiles.
// Weights exp2(s c - m c + 5) then never exceed 2^8 < 448, so their e4m3 rounding cannot
// overflow. S(t) and P(t) alternate between the A and B registers (A for even t).
__device__ __forceinline__ void run(const Ctx& cx, int n_kt, Acc& acc, const i32x8 (&qr)[2], const Lane& ln,
                                    const i32x8& sel) {
  if (n_kt >= 2) {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_tile(cx, t);
  } else {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_tile_short(cx, t);
  }
#pragma unroll
  for (int db = 0; db < 4; ++db) acc.O[db] = f32x16{};
  acc.LB = f32x4{};
  acc.l = 0.f;
  wait_vmcnt<kOpsPerTile * (kAhead - 2)>();
  barrier_lds();
  f32x16 SA[2], SB[2];
  i32x8 PA = {}, PB = {};
  qk_tile(bases(ln, 0, 0), qr, SA);
  if (n_kt == 1) {
    mask_tail(SA, cx.seg_len, ln.h32);
    acc.m = row_max(SA);
    softmax_all(SA, PA, acc.l, cx.c, kRefLog2 - acc.m * cx.c);
    pv_tile(acc, bases(ln, 0, 0), PA, sel);
    wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS past this point
    return;
  }
  acc.m = row_max(SA);
  softmax_all(SA, PA, acc.l, cx.c, kRefLog2 - acc.m * cx.c);
  qk_tile(bases(ln, slot_of(1), 0), qr, SB);
  load_tile(cx, kAhead);
  wait_vmcnt<kOpsPerTile * (kAhead - 3)>();  // as after an odd tile: tiles 2 and 3 are read next
  barrier_lds();

  const int last = n_kt - 2;
  int t = 1;
  // Eight tiles per iteration (ring slots 1..7, 0), then up to seven more.
  for (; t + 7 <= last; t += 8) {
    step<1>(cx, t + 0, acc, SB, SA, PA, PB, qr, ln, sel);
    step<2>(cx, t + 1, acc, SA, SB, PB, PA, qr, ln, sel);
    step<3>(cx, t + 2, acc, SB, SA, PA, PB, qr, ln, sel);
    step<4>(cx, t + 3, acc, SA, SB, PB, PA, qr, ln, sel);
    step<5>(cx, t + 4, acc, SB, SA, PA, PB, qr, ln, sel);
    step<6>(cx, t + 5, acc, SA, SB, PB, PA, qr, ln, sel);
    step<7>(cx, t + 6, acc, SB, SA, PA, PB, qr, ln, sel);
    step<0>(cx, t + 7, acc, SA, SB, PB, PA, qr, ln, sel);
  }
  if (t <= last) step<1>(cx, t, acc, SB, SA, PA, PB, qr, ln, sel);
  if (t + 1 <= last) step<2>(cx, t + 1, acc, SA, SB, PB, PA, qr, ln, sel);
  if (t + 2 <= last) step<3>(cx, t + 2, acc, SB, SA, PA, PB, qr, ln, sel);
  if (t + 3 <= last) step<4>(cx, t + 3, acc, SA, SB, PB, PA, qr, ln, sel);
  if (t + 4 <= last) step<5>(cx, t + 4, acc, SB, SA, PA, PB, qr, ln, sel);
  if (t + 5 <= last) step<6>(cx, t + 5, acc, SA, SB, PB, PA, qr, ln, sel);
  if (t + 6 <= last) step<7>(cx, t + 6, acc, SB, SA, PA, PB, qr, ln, sel);
  if ((n_kt - 1) & 1) last_tile(cx, n_kt, acc, SB, PA, PB, ln, sel);
  else last_tile(cx, n_kt, acc, SA, PB, PA, ln, sel);
  wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS past this point
}

// Keys per range when a segment of seg_len keys is cut into n_split consecutive ranges: whole
// 64-key tiles but for the last range; ranges that start at or past seg_len are empty.
__device__ __forceinline__ int keys_per_split(int seg_len, int n_split) {
  return ((seg_len + n_split - 1) / n_split + kBK - 1) / kBK * kBK;
}

// One workgroup: 256 query rows of one (segment, head) against all keys of the segment; O (bf16)
// and the LSE are written.
//
// With kTail (lsv_attn_fwd_fp8_tail): XCD x owns logical tiles [x P, (x + 1) P), P =
// ceil(n_logical / 8), as in the plain mapping (tiles from n_logical on do not exist). Its first
// P - n_tail / 8 tiles run whole, in the same order; its last n_tail / 8 tiles (its last,
// partial round) are cut into n_split key ranges that run after them on the same XCD. Tail tile
// i = x (n_tail / 8) + r and range s form piece s n_tail + i, which writes its range's
// dequantised, normalised fp32 O and its LSE to row (256 piece + row in tile) of the partial
// buffers.
template <bool kTail>
__device__ __forceinline__ void fp8_body(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k,
                                         const uint8_t* __restrict__ v, uint16_t* __restrict__ o,
                                         float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens, int n_seqs,
                                         int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c,
                                         float dv, int n_logical, int n_tail, int n_split, float* __restrict__ part_o,
                                         float* __restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  // XCD-aware order, as in the BF16 kernel: head-major ranges per XCD.
  int logical, split = 0, piece = -1;
  if (kTail) {
    const int xcd = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;  // this block's place in its XCD's sequence
    const int per_xcd = (n_logical + 7) >> 3;
    const int t = n_tail >> 3;
    if (j < per_xcd - t) {
      logical = xcd * per_xcd + j;
    } else {
      const int jt = j - (per_xcd - t);
      if (jt >= t * n_split) return;
      split = jt / t;
      const int r = jt - split * t;
      logical = xcd * per_xcd + per_xcd - t + r;
      piece = split * n_tail + xcd * t + r;
    }
  } else {
    const int per_xcd = gridDim.x >> 3;
    logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  }
  if (logical >= n_logical) return;
  const int qt = logical % tiles_per_seq;
  const int hs = logical / tiles_per_seq;
  const int seg = hs % n_seqs;
  const int head = hs / n_seqs;
  const int seg_start = cu_seqlens[seg];
  const int seg_end = cu_seqlens[seg + 1];
  if (seg_start < 0 || seg_end < seg_start || (int64_t)seg_end > total_tokens) return;
  const int seg_len = seg_end - seg_start;
  if (seg_len > max_seqlen) return;
  const int q0 = qt * kBQ;
  if (q0 >= seg_len) return;
  int k0 = 0, k_len = seg_len;  // this workgroup's keys: [k0, k0 + k_len) of the segment
  if (kTail && piece >= 0) {
    const int per = keys_per_split(seg_len, n_split);
    k0 = split * per;
    k_len = min(per, seg_len - k0);
    if (k_len <= 0) return;  // an empty range: the combine pass leaves it out
  }
  // Tail launches fix their epilogue destinations here, so that two addresses and a stride stay
  // live through the key loop rather than the output and partial buffers and the indices into
  // them. Row q0 + rr of the tile: O at o_dst + rr * o_stride, LSE at l_dst[rr].
  char* o_dst = nullptr;
  float* l_dst = nullptr;
  int o_stride = 0;
  if (kTail) {
    const int64_t tok0 = (int64_t)seg_start + q0;
    if (piece >= 0) {  // [piece][row in tile][d] and [piece][row in tile]
      o_dst = (char*)(part_o + (int64_t)piece * kBQ * kD);
      o_stride = kD * (int)sizeof(float);
      l_dst = part_lse + (int64_t)piece * kBQ;
    } else {  // the output itself
      o_dst = (char*)(o + (tok0 * n_heads + head) * kD);
      o_stride = n_heads * kD * (int)sizeof(uint16_t);
      l_dst = lse + (int64_t)head * total_tokens + tok0;
    }
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned lds_base = (unsigned)(uintptr_t)(lds_char*)smem_generic;
  Ctx cx;
  cx.lds_copy = lds_base + wave * 1024;
  cx.row_stride = (unsigned)n_heads * kRow8;
  cx.kbase = (const char*)k + ((int64_t)(seg_start + k0) * n_heads + head) * kRow8;
  cx.vbase = (const char*)v + ((int64_t)(seg_start + k0) * n_heads + head) * kRow8;
  {
    const int i = tid & 63;
    cx.crow = 8 * wave + (i >> 3);
    cx.coff = (unsigned)(((i & 7) ^ sw8(cx.crow)) * 16);
    cx.cconst = (unsigned)cx.crow * cx.row_stride + cx.coff;
  }
  cx.seg_len = k_len;  // the key loop sees only this workgroup's key range
  cx.c = c;
  cx.lazy = kLazyLog2 / c;
  const int n_kt = (k_len + kBK - 1) / kBK;

  Lane ln;
  ln.lane = tid & 63;
  ln.h32 = ln.lane >> 5;
  ln.l32 = ln.lane & 31;
  // K rows: lane (key l32 of half a, h32) reads dims 64 c2 + 32 h32 .. +31, i.e. chunks
  // 4 c2 + 2 h32 + sub of row 32 a + l32. The swizzle of row 32 a + l32 does not depend on a,
  // so key half a is the immediate offset 32 a rows.
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int row = ln.l32;
      const int chunk = 4 * c2 + 2 * ln.h32 + sub;
      ln.kaddr[2 * c2 + sub] = lds_base + row * kRow8 + ((chunk ^ sw8(row)) << 4);
    }
  // V^T (d-block db, read r): in 16-lane group (m0, h32) lane L gives the address of row
  // key_of(h32, 8 r + L / 2) = 16 r + 8 (L / 8) + 4 h32 + (L / 2) % 4, columns
  // 32 db + m0 + 8 (L % 2) .. +7; the read returns to lane L column 32 db + m0 + L of those 8
  // rows. The swizzle of that row does not depend on r, so read r is the immediate offset 16 r
  // rows.
  {
    const int L = ln.lane & 15, m0 = 16 * ((ln.lane >> 4) & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int row = key_of(ln.h32, L >> 1);
      const int col = 32 * db + m0 + 8 * (L & 1);
      ln.vaddr[db] = lds_base + kRingBytes + row * kRow8 + (((col >> 4) ^ sw8(row)) << 4) + (col & 15);
    }
  }

  // Q^T operand: lane (query l32, h32) holds dims 64 c2 + 32 h32 .. +31 for c2 = 0, 1.
  i32x8 qr[2];
  {
    int row = q0 + wave * 32 + ln.l32;
    row = row < seg_len ? row : seg_len - 1;
    const uint8_t* qrow = q + ((int64_t)(seg_start + row) * n_heads + head) * kRow8 + 32 * ln.h32;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const u32x4 x = *(const u32x4*)(qrow + 64 * c2);
      const u32x4 y = *(const u32x4*)(qrow + 64 * c2 + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qr[c2][i] = (int)x[i];
        qr[c2][4 + i] = (int)y[i];
      }
    }
  }
  // Selection operand of the weight-sum MFMA: lane (m = lane % 16, block lane / 16) is all
  // e4m3 ones for m = 0 with an even block and m = 4 with an odd block, else zero.
  i32x8 sel;
  {
    const int m = ln.lane & 15, blk = ln.lane >> 4;
    const bool one = (m == 0 && !(blk & 1)) || (m == 4 && (blk & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) sel[i] = one ? (int)kOnes : 0;
  }

  Acc acc;
  run(cx, n_kt, acc, qr, ln, sel);

  // O = dv (P V) / sum(P) -> bf16; LSE = (m c - 5 + log2 l) ln 2. A key range (a tail piece)
  // writes its O in fp32 and its LSE into the partial buffers.
  const float l = pair_sum(acc.l);
  const float lb = pair_sum(acc.LB[0]);  // lanes 32..63 hold 0
  const float mul = dv / lb;
  const int row = q0 + wave * 32 + ln.l32;
  if (row < seg_len) {
    if (kTail && piece >= 0) {
      const int rr = row - q0;
      float* prow = (float*)(o_dst + (int64_t)rr * o_stride);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc.O[db][4 * g + e] * mul;
          *(f32x4*)(prow + 32 * db + 8 * g + 4 * ln.h32) = w;
        }
      if (ln.h32 == 0) l_dst[rr] = (acc.m * c - kRefLog2 + __log2f(l)) * 0.69314718055994530942f;
    } else {
      uint16_t* orow;
      float* lrow;
      if (kTail) {
        orow = (uint16_t*)(o_dst + (int64_t)(row - q0) * o_stride);
        lrow = l_dst + (row - q0);
      } else {
        const int64_t tok = (int64_t)seg_start + row;
        orow = o + (tok * n_heads + head) * kD;
        lrow = lse + (int64_t)head * total_tokens + tok;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x2 lo, hi;
          lo[0] = (__bf16)(acc.O[db][4 * g + 0] * mul);
          lo[1] = (__bf16)(acc.O[db][4 * g + 1] * mul);
          hi[0] = (__bf16)(acc.O[db][4 * g + 2] * mul);
          hi[1] = (__bf16)(acc.O[db][4 * g + 3] * mul);
          u32x2 pk;
          pk[0] = __builtin_bit_cast(unsigned, lo);
          pk[1] = __builtin_bit_cast(unsigned, hi);
          *(u32x2*)(orow + 32 * db + 8 * g + 4 * ln.h32) = pk;
        }
      if (ln.h32 == 0) *lrow = (acc.m * c - kRefLog2 + __log2f(l)) * 0.69314718055994530942f;
    }
  }
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_fp8_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                    uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                    int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c,
                    float dv, int n_logical) {
  fp8_body<false>(q, k, v, o, lse, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, n_heads, total_tokens, c, dv,
                  n_logical, 0, 1, nullptr, nullptr);
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_fp8_tail_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                         uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                         int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c,
                         float dv, int n_logical, int n_tail, int n_split, float* __restrict__ part_o,
                         float* __restrict__ part_lse) {
  fp8_body<true>(q, k, v, o, lse, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, n_heads, total_tokens, c, dv,
                 n_logical, n_tail, n_split, part_o, part_lse);
}

// Merges the key ranges of the tail tiles of attn_fwd_fp8_tail_kernel: block i takes tail tile
// i = x (n_tail / 8) + r, the logical tile x P + P - n_tail / 8 + r (P = ceil(n_logical / 8);
// none from n_logical on), with the forward's segment checks; per row, over the non-empty ranges
// r, LSE = ln sum_r exp(LSE_r) and O = sum_r exp(LSE_r - LSE) O_r in fp32, then bf16 (nearest
// even). 16 lanes per row, 8 dims a lane.
__global__ void __launch_bounds__(256)
attn_fwd_fp8_tail_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                 uint16_t* __restrict__ o, float* __restrict__ lse,
                                 const int32_t* __restrict__ cu_seqlens, int n_seqs, int tiles_per_seq,
                                 int max_seqlen, int n_heads, int64_t total_tokens, int n_logical, int n_tail,
                                 int n_split) {
  const int t = blockIdx.x;
  if (t >= n_tail) return;
  const int per_xcd = (n_logical + 7) >> 3;
  const int tail_per_xcd = n_tail >> 3;
  const int logical = (t / tail_per_xcd + 1) * per_xcd - tail_per_xcd + t % tail_per_xcd;
  if (logical >= n_logical) return;  // past the end of the last XCD's range
  const int qt = logical % tiles_per_seq;
  const int hs = logical / tiles_per_seq;
  const int seg = hs % n_seqs;
  const int head = hs / n_seqs;
  const int seg_start = cu_seqlens[seg];
  const int seg_end = cu_seqlens[seg + 1];
  if (seg_start < 0 || seg_end < seg_start || (int64_t)seg_end > total_tokens) return;
  const int seg_len = seg_end - seg_start;
  if (seg_len > max_seqlen) return;
  const int q0 = qt * kBQ;
  if (q0 >= seg_len) return;
  const int per = keys_per_split(seg_len, n_split);
  const int n_ranges = (seg_len + per - 1) / per;  // the non-empty ranges
  const int j = threadIdx.x & 15;
  const int q_end = min(q0 + kBQ, seg_len);
  for (int row = q0 + (threadIdx.x >> 4); row < q_end; row += 16) {
    const int64_t tok = (int64_t)seg_start + row;
    float m = -INFINITY;
    for (int r = 0; r < n_ranges; ++r) m = fmaxf(m, part_lse[(int64_t)(r * n_tail + t) * kBQ + (row - q0)]);
    float sum = 0.f;
    f32x4 a = {}, b = {};
    for (int r = 0; r < n_ranges; ++r) {
      const int64_t pr = (int64_t)(r * n_tail + t) * kBQ + (row - q0);
      const float w = __expf(part_lse[pr] - m);
      sum += w;
      const f32x4* src = (const f32x4*)(part_o + pr * kD + 8 * j);
      const f32x4 x = src[0], y = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = __builtin_fmaf(w, x[e], a[e]);
        b[e] = __builtin_fmaf(w, y[e], b[e]);
      }
    }
    const float inv = 1.f / sum;
    u32x4 pk;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x2 lo, hi;
      lo[0] = (__bf16)(a[2 * e] * inv);
      lo[1] = (__bf16)(a[2 * e + 1] * inv);
      hi[0] = (__bf16)(b[2 * e] * inv);
      hi[1] = (__bf16)(b[2 * e + 1] * inv);
      pk[e] = __builtin_bit_cast(unsigned, lo);
      pk[2 + e] = __builtin_bit_cast(unsigned, hi);
    }
    *(u32x4*)(o + (tok * n_heads + head) * kD + 8 * j) = pk;
    if (j == 0) lse[(int64_t)head * total_tokens + tok] = m + __logf(sum);
  }
}

constexpr int kProceed = 1;  // fp8_checks: arguments valid and there is work to launch

// The FP8 forward's argument checks (before any HIP call): a status to return, or kProceed with
// the number of 256-row query tiles per segment and c = scale dq dk log2(e).
int fp8_checks(const void* q, const void* k, const void* v, float descale_q, float descale_k, float descale_v,
               const void* o, const float* lse, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
               int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale, int64_t* tiles, float* c) {
  if (n_seqs < 0 || max_seqlen < 0 || total_tokens < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LSV_ERR_INVALID_ARG;
  if (!(descale_q > 0.f) || !(descale_k > 0.f) || !(descale_v > 0.f) || !isfinite(descale_q) ||
      !isfinite(descale_k) || !isfinite(descale_v))
    return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (n_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return LSV_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return LSV_ERR_ALIGNMENT;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return LSV_ERR_ALIGNMENT;
  if (total_tokens > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  const int64_t row_stride = (int64_t)n_heads * kRow8;
  if (row_stride >= (1 << 24) || (int64_t)max_seqlen >= (1 << 24) ||
      (int64_t)max_seqlen * row_stride + kRow8 > (int64_t)UINT32_MAX)
    return LSV_ERR_UNSUPPORTED;
  *tiles = ((int64_t)max_seqlen + kBQ - 1) / kBQ;
  *c = (float)((double)scale * (double)descale_q * (double)descale_k * 1.4426950408889634074);
  if (!(*c > 0.f) || !isfinite(*c)) return LSV_ERR_INVALID_ARG;
  return kProceed;
}

}  // namespace

extern "C" int lsv_attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                                float descale_v, void* o, float* lse, const int32_t* cu_seqlens, int32_t n_seqs,
                                int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                                float scale, void* stream) {
  int64_t tiles = 0;
  float c = 0.f;
  const int rc = fp8_checks(q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens, n_seqs, max_seqlen,
                            total_tokens, n_heads, head_dim, scale, &tiles, &c);
  if (rc != kProceed) return rc;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_fp8_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_fp8_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, (hipStream_t)stream,
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, cu_seqlens,
                     (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads, total_tokens, c, descale_v,
                     (int)n_logical);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

// The plan (lsv_attn_fwd_tail_plan) counts 256-row query tiles and keeps at least 1024 keys per
// range, i.e. whole 64-key tiles here.
static_assert(kBQ == 256 && 1024 % kBK == 0, "the tail plan's tile and range sizes");

extern "C" int lsv_attn_fwd_fp8_tail(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                                     float descale_v, void* o, float* lse, const int32_t* cu_seqlens, int32_t n_seqs,
                                     int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                                     float scale, int32_t compute_units, void* workspace, int64_t workspace_bytes,
                                     void* stream) {
  if (compute_units < 8 || compute_units % 8 != 0) return LSV_ERR_INVALID_ARG;
  int64_t tiles = 0;
  float c = 0.f;
  const int rc = fp8_checks(q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens, n_seqs, max_seqlen,
                            total_tokens, n_heads, head_dim, scale, &tiles, &c);
  if (rc != kProceed) return rc;
  int32_t n_split = 1;
  int64_t n_tail = 0;
  if (lsv_attn_fwd_tail_plan(n_seqs, max_seqlen, n_heads, compute_units, &n_split, &n_tail) != LSV_OK)
    return LSV_ERR_INVALID_ARG;
  if (n_split == 1)
    return lsv_attn_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens, n_seqs, max_seqlen,
                            total_tokens, n_heads, head_dim, scale, stream);
  if (!workspace) return LSV_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 15) return LSV_ERR_ALIGNMENT;
  const int64_t pieces = n_tail * n_split;
  if (workspace_bytes < pieces * kBQ * (kD + 1) * (int64_t)sizeof(float)) return LSV_ERR_INVALID_ARG;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8 - n_tail + pieces;  // 8 x (blocks per XCD)
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_fp8_tail_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  float* part_o = (float*)workspace;
  float* part_lse = part_o + pieces * kBQ * kD;
  const hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_fp8_tail_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st,
                     (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, cu_seqlens,
                     (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads, total_tokens, c, descale_v,
                     (int)n_logical, (int)n_tail, (int)n_split, part_o, part_lse);
  hipLaunchKernelGGL(attn_fwd_fp8_tail_combine_kernel, dim3((unsigned)n_tail), dim3(256), 0, st, part_o, part_lse,
                     (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads,
                     total_tokens, (int)n_logical, (int)n_tail, (int)n_split);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}
