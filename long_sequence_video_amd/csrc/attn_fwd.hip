// Dense non-causal varlen BF16 attention forward for gfx950 (MI355X), with the C ABI.
//
// The operation is the varlen forward of FastVideo #2049 (diff of
// fastvideo/attention/utils/flash_attn_cute.py): per packed segment, head and query row,
// O = softmax(scale * q K^T) V over the keys of the same segment, plus the natural-log
// LSE, non-causal, one split. TensorRT-LLM PR #21275 (Description) gives the shapes this
// kernel is built for: 19k-104k packed tokens, 56 heads (or one sp=4 rank's 14) x 128.
//
// Design (gfx950, wave64):
//  * One workgroup = 8 waves = 256 query rows of one (segment, head), two waves per SIMD
//    (the second wave keeps the VALU issuing while the first waits); each wave owns 32
//    query rows and at most 256 registers.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    A = a 32-key x 16-dim slice of K read from LDS, B = Q^T held in registers for the
//    whole loop. The accumulator then gives every lane one query column and 16 of the
//    32 keys (the other 16 sit in lane l^32), so row max and row sum are in-lane plus
//    one v_permlane32_swap.
//  * O^T += V^T P^T, again 32x32x16: the bf16-converted score accumulator is used as
//    the B operand as is; the MFMA's reduction index is mapped to keys in the
//    accumulator's row order, and V^T is read from row-major V in LDS with
//    ds_read_b64_tr_b16 in that same key order. No shuffles of P.
//  * K and V tiles of 32 keys stream from global memory straight into an 8-slot LDS ring
//    with 16-byte global_load_lds_dwordx4, five tiles ahead of use; one barrier per two tiles.
//    A tile's row offset is uniform (scalar base), so the copies cost no vector ALU; the
//    last, partial tile of a segment is loaded shifted to end at the segment end, and its
//    leading keys (already counted in the previous tile) are masked.
//  * Softmax in the exp2 domain: c = scale * log2(e) is folded into one fp32 FMA per score,
//    p = exp2(s c - m c). The fast path fixes each row's reference m to the max of its
//    first key tile and never moves it: later p may exceed 1, which floating point absorbs
//    unless p overflows, and then the row sums become non-finite. So the steady state
//    carries no max tracking and no O rescale. If any row of the workgroup overflowed, the
//    workgroup recomputes its tile with an exact online softmax (running max, O rescale).
//  * Software pipeline per key tile t: one sequence of 18 MFMAs (O += P(t-1) V(t-1), the two
//    row-sum MFMAs of P(t-1), then S(t+1) = Q K(t+1)^T) with the exp2 work of S(t) placed
//    between them (explicit scheduling barriers hold the order); the steady-state loop body
//    is branch-free.
//  * P V uses p rounded to bf16 and O is divided by the sum of those same rounded p (on the
//    fast path from two small selection MFMAs per tile, which keeps it off the vector ALU:
//    the loop runs at the chip's power limit, so vector work costs matrix issue); the
//    LSE uses the sum of the fp32 p.
//  * LDS: K rows are XOR-swizzled in 16-byte chunks (conflict-free 32-row reads of one
//    chunk); V 4-row blocks are stored column-block first (conflict-free transposing reads,
//    and every V read address is one lane base plus an immediate).
//  * Key-split variant (attn_fwd_split_kernel + attn_fwd_combine_kernel): the same body runs
//    each query tile against one of n consecutive key ranges and writes that range's fp32 O and
//    LSE; a second pass merges them per row. More, shorter workgroups fill the last round of
//    compute units when a launch has few query tiles.
//  * Workgroups are remapped so that consecutive tiles of one (head, segment) land on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2; each XCD's range is
//    head-major (heads spread evenly over the XCDs), segments in packed order.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "lsv.h"
#include "tile_ops.h"

namespace {

using namespace lsv_tiles;

constexpr int kD = 128;                       // head dim
constexpr int kWaveQ = 32;                    // query rows per wave
constexpr int kWaves = 8;                     // waves per workgroup
constexpr int kBQ = kWaveQ * kWaves;          // query rows per workgroup
constexpr int kBK = 32;                       // keys per tile
constexpr int kSlots = 8;                     // LDS ring slots (K and V each)
constexpr int kAhead = 5;                     // tiles in flight ahead of use
constexpr int kThreads = kWaves * 64;
constexpr int kSlotBytes = kTileBytes;        // 8 KB: 32 key rows of 256 bytes
constexpr int kRingBytes = kSlots * kSlotBytes;
constexpr int kLdsBytes = 2 * kRingBytes + 64;  // K ring, V ring (128 KB), workgroup flags
constexpr int kCopies = kSlotBytes / 1024 / kWaves;  // 1 KB copies per wave per tile, for K and for V
constexpr int kOpsPerTile = 2 * kCopies;             // memory instructions per wave per tile
constexpr float kLazyLog2 = 8.0f;             // exact path: raise the running max only beyond this
static_assert(kCopies == 1, "one 1 KB copy per wave per tile");
// The workgroup synchronises after odd tiles only. Between two barriers a wave runs at most
// tiles t+1, t+2 (t odd) and copies tiles t+1+kAhead, t+2+kAhead, into the slots of tiles
// t+1+kAhead-kSlots and t+2+kAhead-kSlots; a wave still behind has finished tile t, so it may
// read V(t), K(t+2) (tile t+1) or V(t+1), K(t+3) (tile t+2): the written slots must be none
// of tiles t .. t+3, i.e. kAhead <= kSlots - 3. Each barrier follows the wait for tile t+3
// (read as K by tile t+2), leaving kAhead - 3 tiles in flight.
static_assert(kAhead >= 3 && kAhead <= kSlots - 3, "ring too small for the prefetch distance");

struct Lane {
  int lane, h32, l32;
  unsigned kaddr[8];  // K-ring LDS address of 16-dim step s in slot 0 (slot offsets are immediates)
  unsigned vaddr;     // V-ring LDS address of this lane's transposed read (d-block 0, key half 0,
                      // slot 0); the others are immediate offsets from it
};

struct Ctx {
  unsigned lds_copy;    // LDS byte address of this wave's 1 KB part of ring slot 0 (wave-uniform)
  const char* kbase;    // k row `seg_start`, this head (wave-uniform)
  const char* vbase;
  unsigned row_stride;  // bytes between token rows (< 2^24)
  int krow, vrow;       // the tile row this lane copies, for K and for V
  unsigned koff, voff;  // the byte offset inside that row
  int seg_len;
  float c;              // scale * log2(e)
  unsigned kconst, vconst;  // krow * row_stride + koff, vrow * row_stride + voff
};

// Per-lane softmax state (query row l32, this lane's 16 of every 32 keys).
struct Acc {
  f32x16 O[4];  // O^T accumulator, d-block db
  float m;      // reference max (raw score units)
  float l;      // sum of fp32 p: for the LSE
  float lb;     // sum of bf16(p), the weights P V used: normalises O
  f32x4 LBm;    // fast path: element 0 of lanes 0..31 = sum of bf16(p) of query l32
};

// Row sums of bf16 P: one v_mfma_f32_16x16x32_bf16 per P operand whose A selects, for output
// row 0, the lanes of queries 0..15 (lane blocks 0 and 2 of B) and, for row 4, those of
// queries 16..31 (blocks 1 and 3). Row 0 lands in element 0 of lanes 0..15 and row 4 in
// element 0 of lanes 16..31: each sum in the lane whose l32 is its query (lanes 32..63 get 0).
__device__ __forceinline__ f32x4 mfma_rowsum(const bf16x8& sel, const bf16x8& p, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p, c, 0, 0, 0);
}

// Tile copies. Wave w copies rows 4w .. 4w+3 of the 32-row tile of K and of V (1 KB
// apiece) into the ring slot at byte offset `slot`; lane i writes 16-byte slot i of that
// block:
//   K block: slot i holds row 4w + i / 16, chunk (i % 16) ^ swz(row)   (XOR swizzle)
//   V block: slot i holds row 4w + (i / 4) % 4, chunk 4 (i / 16) + i % 4 (column-block
//            order: the 16 chunks of one 32-dim block of the 4 rows are contiguous)
//
// Segments of 32 keys or more: tile t holds rows min(32 t, seg_len - 32) .. +31, all inside
// the segment (the last tile is shifted back to end at the segment end; tiles past the end,
// which are prefetched but never used, repeat it). The row offset is uniform and goes into
// the scalar base address; the lane's offset is a constant.
__device__ __forceinline__ void load_tile_shifted(const Ctx& cx, int t, unsigned slot) {
  const int start = min(t * kBK, cx.seg_len - kBK);
  const unsigned off = (unsigned)start * cx.row_stride;
  dma16(cx.kconst, cx.kbase + off, cx.lds_copy + slot);
  dma16(cx.vconst, cx.vbase + off, cx.lds_copy + slot + kRingBytes);
}

// Segments shorter than 32 keys (a single tile): rows past the segment repeat its last row.
__device__ __forceinline__ void load_tile_to(const Ctx& cx, int t, unsigned slot) {
  const int tkey = t * kBK, last = cx.seg_len - 1;
  const int kkey = tkey + cx.krow < last ? tkey + cx.krow : last;
  const int vkey = tkey + cx.vrow < last ? tkey + cx.vrow : last;
  dma16(__umul24((unsigned)kkey, cx.row_stride) + cx.koff, cx.kbase, cx.lds_copy + slot);
  dma16(__umul24((unsigned)vkey, cx.row_stride) + cx.voff, cx.vbase, cx.lds_copy + slot + kRingBytes);
}

// Tile t into its ring slot t % kSlots (segments of 32 keys or more).
__device__ __forceinline__ void load_tile(const Ctx& cx, int t) {
  load_tile_shifted(cx, t, (unsigned)(t & (kSlots - 1)) * kSlotBytes);
}

// S^T (32 keys x 32 queries) = K(slot) Q^T: 8 MFMAs over the 128 dims.
__device__ __forceinline__ f32x16 qk_tile(unsigned slot, const bf16x8 (&qr)[8], const Lane& ln) {
  f32x16 S = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) S = mfma(lds_row(ln.kaddr[s] + slot), qr[s], S);
  return S;
}

// O^T (128 dims x 32 queries) += V(slot)^T P^T: 2 key chunks of 16 x 4 d-blocks of 32.
__device__ __forceinline__ void pv_tile(f32x16 (&O)[4], unsigned slot, const bf16x8 (&P)[2], const Lane& ln) {
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i & 3] = mfma(tr_operand(ln.vaddr, slot, i), P[i >> 2], O[i & 3]);
}

// Keys at and past `valid` in the tile are outside the segment: element v of S holds key
// 8 (v / 4) + 4 h32 + v % 4.
__device__ __forceinline__ void mask_tail(f32x16& S, int valid, const Lane& ln) {
  const int lim = valid - 4 * ln.h32;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (8 * (v >> 2) + (v & 3) >= lim) S[v] = -INFINITY;
}

// The shifted last tile: its first `skip` keys were already counted in the tile before.
__device__ __forceinline__ void mask_head(f32x16& S, int skip, const Lane& ln) {
  const int lim = skip - 4 * ln.h32;
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (8 * (v >> 2) + (v & 3) < lim) S[v] = -INFINITY;
}

// This lane's max over its 16 scores of the tile.
__device__ __forceinline__ float lane_max(const f32x16& S) {
  float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, S[v]), S[v + 1]);
  return fmaxf(mx, S[15]);
}

// Scores 2j, 2j+1: p = exp2(s c - m c) -> bf16 pair into P; row sum of the fp32 p (l) and,
// on the exact path (kLb), of the bf16 p (lb, v_dot2_f32_bf16). The fast path sums the bf16 p
// with row-sum MFMAs instead (mfma_rowsum), off the vector ALU.
template <bool kLb = true>
__device__ __forceinline__ void softmax_pair(const f32x16& S, u32x4 (&P)[2], float& l, float& lb, float c,
                                             float nmc, int j) {
  const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * j], c, nmc));
  const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * j + 1], c, nmc));
  l += e0;
  l += e1;
  bf16x2 pp, one;
  pp[0] = (__bf16)e0;
  pp[1] = (__bf16)e1;
  one[0] = (__bf16)1.0f;
  one[1] = (__bf16)1.0f;
  if (kLb) lb = __builtin_amdgcn_fdot2_f32_bf16(pp, one, lb, false);
  P[j >> 2][j & 3] = __builtin_bit_cast(unsigned, pp);
}

template <bool kLb = true>
__device__ __forceinline__ void softmax_all(const f32x16& S, bf16x8 (&P)[2], float& l, float& lb, float c,
                                            float nmc) {
  u32x4 p[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) softmax_pair<kLb>(S, p, l, lb, c, nmc, j);
  P[0] = __builtin_bit_cast(bf16x8, p[0]);
  P[1] = __builtin_bit_cast(bf16x8, p[1]);
}

// ---------------------------------------------------------------------------- fast path

// Steady-state tile t (1 <= t <= n_kt - 2, t % kSlots == U): one sequence of 16 MFMAs,
//   n = 0..7:  O += P(t-1) V(t-1)   (V operand n), then after n = 7 the two row-sum MFMAs
//              of P(t-1)
//   n = 8..15: S(t+1) = Q K(t+1)^T  (K operand n - 8)
// with each LDS operand read two MFMAs ahead, the eight exp2 pairs of S(t) after the odd
// MFMAs, and the copy of tile t + kAhead after MFMA 4. After an odd tile, tile t+3 is waited
// for and the workgroup synchronises. No branches.
constexpr int kReadAhead = 3;  // LDS operands are read this many MFMAs ahead of their use

template <int U>
__device__ __forceinline__ void fast_step(const Ctx& cx, int t, Acc& acc, const f32x16& Scur, f32x16& Snext,
                                          const bf16x8 (&Pprev)[2], bf16x8 (&Pcur)[2], float nmc,
                                          const bf16x8 (&qr)[8], const Lane& ln, const bf16x8& sel) {
  constexpr unsigned vslot = ((U + kSlots - 1) % kSlots) * kSlotBytes;
  constexpr unsigned kslot = ((U + 1) % kSlots) * kSlotBytes;
  bf16x8 opnd[16];
  auto read = [&](int n) {
    if (n < 8) opnd[n] = tr_operand(ln.vaddr, vslot, n);
    else opnd[n] = lds_row(ln.kaddr[n - 8] + kslot);
  };
#pragma unroll
  for (int n = 0; n < kReadAhead; ++n) read(n);
  sched_fence();
  u32x4 p[2];
  f32x16 S = {};
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    if (n < 8) acc.O[n & 3] = mfma(opnd[n], Pprev[n >> 2], acc.O[n & 3]);
    else S = mfma(opnd[n], qr[n - 8], S);
    if (n + kReadAhead < 16) read(n + kReadAhead);
    if (n == 4) load_tile(cx, t + kAhead);
    if (n == 7) {
      acc.LBm = mfma_rowsum(sel, Pprev[0], acc.LBm);
      acc.LBm = mfma_rowsum(sel, Pprev[1], acc.LBm);
    }
    if (n & 1) softmax_pair<false>(Scur, p, acc.l, acc.lb, cx.c, nmc, n >> 1);
    sched_fence();
  }
  Snext = S;
  Pcur[0] = __builtin_bit_cast(bf16x8, p[0]);
  Pcur[1] = __builtin_bit_cast(bf16x8, p[1]);
  // P(t) and the row sums must be complete here (they must not sink into the next tile).
  asm volatile("" : "+v"(Pcur[0]), "+v"(Pcur[1]), "+v"(acc.l), "+v"(acc.lb));
  if (U & 1) {
    wait_vmcnt<kOpsPerTile * (kAhead - 3)>();
    barrier_lds();
  }
}

// Row sums of the bf16 P of one tile (fast path, outside the pipelined steps).
__device__ __forceinline__ void lb_tile(Acc& acc, const bf16x8& sel, const bf16x8 (&P)[2]) {
  acc.LBm = mfma_rowsum(sel, P[0], acc.LBm);
  acc.LBm = mfma_rowsum(sel, P[1], acc.LBm);
}

// Runs the whole key loop with a fixed per-row reference (the max of the first tile).
// Returns false when any of this lane's sums or O values is not finite (inf or NaN: a p
// overflowed, or two overflowed products of opposite sign met in one O element).
// The first kAhead tile copies of the key loop.
__device__ __forceinline__ void prefetch(const Ctx& cx, int n_kt) {
  if (n_kt >= 2) {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_tile(cx, t);
  } else {  // one tile of fewer than 32 keys (32 exactly is the same either way)
#pragma unroll
    for (int t = 0; t < kAhead; ++t) load_tile_to(cx, t, (unsigned)t * kSlotBytes);
  }
}

// With kPrefetched, the caller has issued prefetch() already.
template <bool kPrefetched = false>
__device__ __forceinline__ bool run_fast(const Ctx& cx, int n_kt, Acc& acc, const bf16x8 (&qr)[8],
                                         const Lane& ln, const bf16x8& sel) {
  if (!kPrefetched) prefetch(cx, n_kt);
  wait_vmcnt<kOpsPerTile * (kAhead - 2)>();
  barrier_lds();
#pragma unroll
  for (int db = 0; db < 4; ++db) acc.O[db] = f32x16{};
  acc.l = 0.f;
  acc.lb = 0.f;
  acc.LBm = f32x4{};
  f32x16 SA, SB;
  bf16x8 PA[2], PB[2];

  // Tile 0 sets the reference.
  SA = qk_tile(0, qr, ln);
  if (n_kt == 1) mask_tail(SA, cx.seg_len, ln);
  acc.m = pair_max(lane_max(SA));
  const float nmc = -acc.m * cx.c;
  softmax_all<false>(SA, PA, acc.l, acc.lb, cx.c, nmc);
  if (n_kt > 1) {
    SB = qk_tile(1 * kSlotBytes, qr, ln);
    load_tile(cx, kAhead);
    wait_vmcnt<kOpsPerTile * (kAhead - 3)>();  // as after an odd tile: tiles 2 and 3 are read next
    barrier_lds();
  }

  // Tiles 1 .. n_kt-2: eight per iteration (slots 1..7, 0), then up to seven more.
  // S(t) is in SA for even t, SB for odd t; P(t) likewise in PA / PB.
  const int last = n_kt - 2;
  int t = 1;
  for (; t + 7 <= last; t += 8) {
    fast_step<1>(cx, t + 0, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
    fast_step<2>(cx, t + 1, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
    fast_step<3>(cx, t + 2, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
    fast_step<4>(cx, t + 3, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
    fast_step<5>(cx, t + 4, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
    fast_step<6>(cx, t + 5, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
    fast_step<7>(cx, t + 6, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
    fast_step<0>(cx, t + 7, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
  }
  if (t <= last) fast_step<1>(cx, t, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
  if (t + 1 <= last) fast_step<2>(cx, t + 1, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
  if (t + 2 <= last) fast_step<3>(cx, t + 2, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
  if (t + 3 <= last) fast_step<4>(cx, t + 3, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
  if (t + 4 <= last) fast_step<5>(cx, t + 4, acc, SB, SA, PA, PB, nmc, qr, ln, sel);
  if (t + 5 <= last) fast_step<6>(cx, t + 5, acc, SA, SB, PB, PA, nmc, qr, ln, sel);
  if (t + 6 <= last) fast_step<7>(cx, t + 6, acc, SB, SA, PA, PB, nmc, qr, ln, sel);

  // Last tile (n_kt >= 2): P V of tile n_kt-2, masked exp2 of the shifted tile n_kt-1, its P V.
  const int tl = n_kt - 1;
  if (tl >= 1) {
    const unsigned vprev = ((tl - 1) & (kSlots - 1)) * kSlotBytes;
    const unsigned vlast = (tl & (kSlots - 1)) * kSlotBytes;
    const int skip = kBK - (cx.seg_len - tl * kBK);
    if (tl & 1) {
      pv_tile(acc.O, vprev, PA, ln);
      lb_tile(acc, sel, PA);
      mask_head(SB, skip, ln);
      softmax_all<false>(SB, PB, acc.l, acc.lb, cx.c, nmc);
      pv_tile(acc.O, vlast, PB, ln);
      lb_tile(acc, sel, PB);
    } else {
      pv_tile(acc.O, vprev, PB, ln);
      lb_tile(acc, sel, PB);
      mask_head(SA, skip, ln);
      softmax_all<false>(SA, PA, acc.l, acc.lb, cx.c, nmc);
      pv_tile(acc.O, vlast, PA, ln);
      lb_tile(acc, sel, PA);
    }
  } else {
    pv_tile(acc.O, 0, PA, ln);
    lb_tile(acc, sel, PA);
  }
  acc.lb = acc.LBm[0];  // lanes 32..63 hold 0: the epilogue's pair sum is the row's sum
  // No copy may still be writing this workgroup's LDS past this point.
  wait_vmcnt<0>();
  // Finite check of l, lb and all 64 O values on their bit patterns: a float is inf or NaN
  // exactly when its magnitude bits are at least 0x7f800000, and magnitudes order like their
  // bit patterns, so the integer max over all of them decides. (A float max would drop a NaN,
  // e.g. an O element that received +inf and -inf from two late keys while l stayed finite.)
  // The magnitude bits are taken in asm, so that nothing the build's no-NaN setting lets the
  // compiler assume about the floats can fold the test away.
  unsigned mag = 0;
  auto fold = [&mag](float x) {
    unsigned u;
    asm("v_and_b32 %0, 0x7fffffff, %1" : "=v"(u) : "v"(x));
    mag = max(mag, u);
  };
  fold(acc.l);
  fold(acc.lb);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) fold(acc.O[db][v]);
  return mag < 0x7f800000u;
}

// ---------------------------------------------------------------------------- exact path

// Exact online softmax, one tile at a time through ring slot 0 (used only when the fast
// path overflowed): running row max with a lazy margin and O rescale; unpipelined.
__device__ __forceinline__ void run_exact(const Ctx& cx, int n_kt, Acc& acc, const bf16x8 (&qr)[8],
                                          const Lane& ln) {
#pragma unroll
  for (int db = 0; db < 4; ++db) acc.O[db] = f32x16{};
  acc.m = -INFINITY;
  acc.l = 0.f;
  acc.lb = 0.f;
  const float lazy = kLazyLog2 / cx.c;
  for (int t = 0; t < n_kt; ++t) {
    barrier_lds();  // every wave is done with slot 0
    if (n_kt >= 2) load_tile_shifted(cx, t, 0);
    else load_tile_to(cx, t, 0);
    wait_vmcnt<0>();
    barrier_lds();
    f32x16 S = qk_tile(0, qr, ln);
    if (t == n_kt - 1) {
      if (n_kt >= 2) mask_head(S, kBK - (cx.seg_len - t * kBK), ln);
      else mask_tail(S, cx.seg_len, ln);
    }
    const float mx = pair_max(lane_max(S));
    if (__builtin_amdgcn_ballot_w64(mx > acc.m + lazy) != 0) {  // wave-uniform
      const float mnew = fmaxf(acc.m, mx);
      const float a = __builtin_amdgcn_exp2f((acc.m - mnew) * cx.c);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc.O[db][v] *= a;
      acc.l *= a;
      acc.lb *= a;
      acc.m = mnew;
    }
    bf16x8 P[2];
    softmax_all(S, P, acc.l, acc.lb, cx.c, -acc.m * cx.c);
    pv_tile(acc.O, 0, P, ln);
  }
  barrier_lds();
}

// Keys per split when a segment of seg_len keys is cut into n_split consecutive ranges: a
// multiple of the key tile, so that every range but the last is whole tiles. Ranges that
// start at or past seg_len are empty.
__device__ __forceinline__ int keys_per_split(int seg_len, int n_split) {
  return ((seg_len + n_split - 1) / n_split + kBK - 1) / kBK * kBK;
}

// The Q-side prologue of lsv_attn_fwd_qnorm: raw q rows are RMS-normalised with weight w and
// rotated (rotate-half RoPE on the first R channels, one cos/sin table row per token) as the
// Q tile is loaded.
struct QNorm {
  const uint16_t* w;    // bf16 [128]
  const uint16_t* cos;  // bf16 [total_tokens, R]
  const uint16_t* sin;
  int r;                // rotary width R, a multiple of 16 in [0, 128]
  float eps;
};

__device__ __forceinline__ void unpack8(const u32x4& u, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

// This lane's Q^T operand from the raw row at `qrow` (token `tok`): chunk s holds channels
// 16 s + 8 h32 .. +7. The arithmetic is the standalone prologue's, step for step, so the operand
// is bit-identical to what that pass would have written: per 8-channel chunk an fma chain of
// squares; the 16 chunk sums of the row added in the same tree (chunk j = 2 s + h32 with
// j ^ 8, j ^ 4, j ^ 2 -- the same lane -- then j ^ 1, the partner lane l ^ 32);
// inv = rsq(ss / 128 + eps); y = x inv w; a rotated channel i is fma(y_p, -+sin_i, y_i cos_i)
// with partner channel p = i +- R/2 (its raw chunk read again from the row); one rounding to bf16.
__device__ __forceinline__ void load_q_normed(const char* qrow, int64_t tok, int h32, const QNorm& qn,
                                              bf16x8 (&qr)[8]) {
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) unpack8(*(const u32x4*)(qrow + 32 * s + 16 * h32), x[s]);
  float p[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = __builtin_fmaf(x[s][e], x[s][e], a);
    p[s] = a;
  }
  float t1[4], t2[2];
#pragma unroll
  for (int s = 0; s < 4; ++s) t1[s] = p[s] + p[s + 4];
  t2[0] = t1[0] + t1[2];
  t2[1] = t1[1] + t1[3];
  const float ss = pair_sum(t2[0] + t2[1]);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + qn.eps);
  const int half = qn.r >> 1;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int i0 = 16 * s + 8 * h32;  // first channel of this chunk
    float w[8];
    unpack8(*(const u32x4*)(qn.w + i0), w);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = x[s][e] * inv * w[e];
    if (i0 < qn.r) {
      const int ip = i0 < half ? i0 + half : i0 - half;
      const float sgn = i0 < half ? -1.0f : 1.0f;
      float xp[8], wp[8], cs[8], sn[8];
      unpack8(*(const u32x4*)(qrow + 2 * ip), xp);
      unpack8(*(const u32x4*)(qn.w + ip), wp);
      unpack8(*(const u32x4*)(qn.cos + tok * qn.r + i0), cs);
      unpack8(*(const u32x4*)(qn.sin + tok * qn.r + i0), sn);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yp = xp[e] * inv * wp[e];
        o[e] = __builtin_fmaf(yp, sgn * sn[e], o[e] * cs[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[s][e] = (__bf16)o[e];
  }
}

// One workgroup: 256 query rows of one (segment, head) against all keys of the segment, or,
// with kSplit, against key range `split` of n_split; then O (bf16) and LSE are written, or,
// with kSplit, this range's normalised fp32 O and its LSE into the partial buffers.
//
// With kTail (lsv_attn_fwd_tail, and lsv_attn_fwd with n_tail = 0; n_tail a multiple of 8):
// XCD x owns logical tiles [x P, (x + 1) P), P = ceil(n_logical / 8), exactly as in the plain
// mapping (tiles from n_logical on do not exist). Its first P - n_tail / 8 tiles run whole, in
// the same order as there; its last n_tail / 8 tiles (its last, partial round) are cut into
// n_split key ranges and run after them, on the same XCD. Tail tile i = x * (n_tail / 8) + r
// and range s form piece s * n_tail + i, which writes its range's fp32 O and LSE to row
// (piece * 256 + row in tile) of the partial buffers.
template <bool kSplit, bool kQNorm = false, bool kTail = false>
__device__ __forceinline__ void fwd_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                                         float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens, int n_seqs,
                                         int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens,
                                         float c, int n_logical, int n_split, float* __restrict__ part_o,
                                         float* __restrict__ part_lse, QNorm qn = QNorm{}, int n_tail = 0) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];

  // XCD-aware order: hardware dispatches block b to XCD b % 8; give each XCD a contiguous
  // range of logical tiles (head-major, then segment in packed order, then key range, then
  // query tile).
  int logical, split = 0, piece = -1;
  if (kTail) {
    const int xcd = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;  // this block's place in its XCD's sequence
    // Each XCD owns ceil(n_logical / 8) consecutive tiles; when n_logical is not a multiple of
    // 8 the last XCD's range runs past the end, and those tiles (whole or cut) do not exist.
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
    if (logical >= n_logical) return;
  } else {
    const int per_xcd = gridDim.x >> 3;
    logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= n_logical) return;
  }
  const int qt = logical % tiles_per_seq;
  int hs = logical / tiles_per_seq;
  if (kSplit) {
    split = hs % n_split;
    hs /= n_split;
  }
  const int seg = hs % n_seqs;
  const int head = hs / n_seqs;
  const int seg_start = cu_seqlens[seg];
  const int seg_end = cu_seqlens[seg + 1];
  if (seg_start < 0 || seg_end < seg_start || (int64_t)seg_end > total_tokens) return;
  const int seg_len = seg_end - seg_start;
  if (seg_len > max_seqlen) return;  // breaks the contract; 32-bit copy offsets assume <= max_seqlen
  const int q0 = qt * kBQ;
  if (q0 >= seg_len) return;
  int k0 = 0, k_len = seg_len;  // this workgroup's keys: [k0, k0 + k_len) of the segment
  if (kSplit || (kTail && piece >= 0)) {
    const int per = keys_per_split(seg_len, n_split);
    k0 = split * per;
    k_len = min(per, seg_len - k0);
    if (k_len <= 0) return;  // an empty range: the combine pass leaves it out
  }

  // Epilogue destinations, fixed here so that two addresses and a stride stay live through the
  // key loop rather than the output buffers and the indices into them (with the split and tail
  // variants' partial buffers as well, that spilled). Row q0 + rr of the tile: O at
  // o_dst + rr * o_stride, LSE at l_dst[rr].
  char* o_dst;
  float* l_dst;
  int o_stride;
  {
    const int64_t tok0 = (int64_t)seg_start + q0;
    if (kSplit) {  // [split][token][head][d] and [split][head][token]
      o_dst = (char*)(part_o + (((int64_t)split * total_tokens + tok0) * n_heads + head) * kD);
      o_stride = n_heads * kD * (int)sizeof(float);
      l_dst = part_lse + ((int64_t)split * n_heads + head) * total_tokens + tok0;
    } else if (kTail && piece >= 0) {  // [piece][row in tile][d] and [piece][row in tile]
      o_dst = (char*)(part_o + (int64_t)piece * kBQ * kD);
      o_stride = kD * (int)sizeof(float);
      l_dst = part_lse + (int64_t)piece * kBQ;
    } else {  // the output itself
      o_dst = (char*)(o + (tok0 * n_heads + head) * kD);
      o_stride = n_heads * kRowBytes;
      l_dst = lse + (int64_t)head * total_tokens + tok0;
    }
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned lds_base = (unsigned)(uintptr_t)(lds_char*)smem_generic;
  Ctx cx;
  cx.lds_copy = lds_base + wave * kCopies * 1024;
  cx.row_stride = (unsigned)n_heads * kRowBytes;
  cx.kbase = (const char*)k + ((int64_t)(seg_start + k0) * n_heads + head) * kRowBytes;
  cx.vbase = (const char*)v + ((int64_t)(seg_start + k0) * n_heads + head) * kRowBytes;
  {
    const int i = tid & 63;
    row_copy_lane(wave, i, cx.krow, cx.koff);  // K: row layout
    tr_copy_lane(wave, i, cx.vrow, cx.voff);   // V: transposed-read layout
    cx.kconst = (unsigned)cx.krow * cx.row_stride + cx.koff;
    cx.vconst = (unsigned)cx.vrow * cx.row_stride + cx.voff;
  }
  cx.seg_len = k_len;  // the key loop sees only this workgroup's key range
  cx.c = c;
  const int n_kt = (k_len + kBK - 1) / kBK;

  Lane ln;
  ln.lane = tid & 63;
  ln.h32 = ln.lane >> 5;
  ln.l32 = ln.lane & 31;
#pragma unroll
  for (int s = 0; s < 8; ++s) ln.kaddr[s] = row_read_addr(lds_base, ln.l32, ln.h32, s);
  ln.vaddr = tr_read_base(lds_base + kRingBytes, ln.lane);

  // Q^T operand: lane holds q[row][16 s + 8 h32 .. +7] for s = 0..7 (normalised and rotated
  // on the way in for lsv_attn_fwd_qnorm, whose key tiles are requested first so that their
  // latency overlaps the Q loads and the normalisation).
  if (kQNorm) prefetch(cx, n_kt);
  bf16x8 qr[8];
  {
    int row = q0 + wave * kWaveQ + ln.l32;
    row = row < seg_len ? row : seg_len - 1;
    const char* qrow = (const char*)q + ((int64_t)(seg_start + row) * n_heads + head) * kRowBytes;
    if (kQNorm) {
      load_q_normed(qrow, (int64_t)seg_start + row, ln.h32, qn, qr);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qr[s] = *(const bf16x8*)(qrow + ln.h32 * 16 + s * 32);
    }
  }

  Acc acc;
  bf16x8 sel;
  {
    const int m = ln.lane & 15, blk = ln.lane >> 4;
    const bool one = (m == 0 && !(blk & 1)) || (m == 4 && (blk & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) sel[i] = one ? (__bf16)1.0f : (__bf16)0.0f;
  }
  const bool ok = run_fast<kQNorm>(cx, n_kt, acc, qr, ln, sel);
  // Workgroup-wide verdict: any overflowing row sends the whole workgroup down the exact path.
  lds_int* flags = (lds_int*)(uintptr_t)(lds_base + 2 * kRingBytes);
  if (tid < kWaves) flags[tid] = 0;
  barrier_lds();
  if (__builtin_amdgcn_ballot_w64(!ok) != 0 && ln.lane == 0) flags[wave] = 1;
  barrier_lds();
  int bad = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) bad |= flags[w];
  if (bad) run_exact(cx, n_kt, acc, qr, ln);

  // Epilogue: O / lb -> bf16, LSE = (m c + log2 l) ln 2; for a key range (kSplit, or a tail
  // piece), O / lb in fp32 and the range's LSE into the partial buffers.
  const float l = pair_sum(acc.l);
  const float lb = pair_sum(acc.lb);
  const int row = q0 + wave * kWaveQ + ln.l32;
  if (row < seg_len) {
    const float lse_row = (acc.m * c + __log2f(l)) * 0.69314718055994530942f;
    const int rr = row - q0;
    if (kSplit || (kTail && piece >= 0)) {
      float* prow = (float*)(o_dst + (int64_t)rr * o_stride);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = acc.O[db][4 * g + e] / lb;
          *(f32x4*)(prow + 32 * db + 8 * g + 4 * ln.h32) = w;
        }
      if (ln.h32 == 0) l_dst[rr] = lse_row;
    } else {
      uint16_t* orow = (uint16_t*)(o_dst + (int64_t)rr * o_stride);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x2 lo, hi;
          lo[0] = (__bf16)(acc.O[db][4 * g + 0] / lb);
          lo[1] = (__bf16)(acc.O[db][4 * g + 1] / lb);
          hi[0] = (__bf16)(acc.O[db][4 * g + 2] / lb);
          hi[1] = (__bf16)(acc.O[db][4 * g + 3] / lb);
          u32x2 pk;
          pk[0] = __builtin_bit_cast(unsigned, lo);
          pk[1] = __builtin_bit_cast(unsigned, hi);
          *(u32x2*)(orow + 32 * db + 8 * g + 4 * ln.h32) = pk;
        }
      if (ln.h32 == 0) l_dst[rr] = lse_row;
    }
  }
}

// The fused-Q forward, with the tail kernel's mapping: n_tail = 0 (lsv_attn_fwd_qnorm) runs every
// tile whole, in the plain launch's XCDs and order.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_qnorm_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                      int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c,
                      int n_logical, QNorm qn, int n_tail, int n_split, float* __restrict__ part_o,
                      float* __restrict__ part_lse) {
  fwd_body<false, true, true>(q, k, v, o, lse, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, n_heads, total_tokens,
                              c, n_logical, n_split, part_o, part_lse, qn, n_tail);
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens, int n_seqs,
                      int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c, int n_logical,
                      int n_split, float* __restrict__ part_o, float* __restrict__ part_lse) {
  fwd_body<true>(q, k, v, nullptr, nullptr, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, n_heads, total_tokens, c,
                 n_logical, n_split, part_o, part_lse);
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_tail_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                     int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens, float c,
                     int n_logical, int n_tail, int n_split, float* __restrict__ part_o, float* __restrict__ part_lse) {
  fwd_body<false, false, true>(q, k, v, o, lse, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, n_heads, total_tokens,
                               c, n_logical, n_split, part_o, part_lse, QNorm{}, n_tail);
}

// Combines the key ranges of the tail tiles of attn_fwd_tail_kernel: block i takes tail tile
// i = x * (n_tail / 8) + r, the logical tile x P + P - n_tail / 8 + r (P = ceil(n_logical / 8);
// none from n_logical on), and merges its rows' ranges as attn_fwd_combine_kernel does (the
// same segment checks; empty ranges left out; fp32, then bf16 nearest even).
__global__ void __launch_bounds__(256)
attn_fwd_tail_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                             uint16_t* __restrict__ o, float* __restrict__ lse,
                             const int32_t* __restrict__ cu_seqlens, int n_seqs, int tiles_per_seq, int max_seqlen,
                             int n_heads, int64_t total_tokens, int n_logical, int n_tail, int n_split) {
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
  const int n_ranges = (seg_len + per - 1) / per;
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

// Combines the key ranges of attn_fwd_split_kernel: per (token, head) row, with LSE_s of the
// non-empty ranges s, LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s (fp32), then
// O -> bf16 (nearest even). One workgroup of 256 threads per (head, segment, 256-row query
// tile), in the forward's order and with its segment checks; 16 lanes per row, 8 dims a lane.
__global__ void __launch_bounds__(256)
attn_fwd_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                        uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                        int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads, int64_t total_tokens,
                        int n_logical, int n_split) {
  const int logical = blockIdx.x;
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
  const int per = keys_per_split(seg_len, n_split);
  const int n_ranges = (seg_len + per - 1) / per;  // the non-empty ranges
  const int j = threadIdx.x & 15;
  const int q_end = min(q0 + kBQ, seg_len);
  for (int row = q0 + (threadIdx.x >> 4); row < q_end; row += 16) {
    const int64_t tok = (int64_t)seg_start + row;
    float m = -INFINITY;
    for (int r = 0; r < n_ranges; ++r) m = fmaxf(m, part_lse[((int64_t)r * n_heads + head) * total_tokens + tok]);
    float sum = 0.f;
    f32x4 a = {}, b = {};
    for (int r = 0; r < n_ranges; ++r) {
      const float w = __expf(part_lse[((int64_t)r * n_heads + head) * total_tokens + tok] - m);
      sum += w;
      const f32x4* src = (const f32x4*)(part_o + (((int64_t)r * total_tokens + tok) * n_heads + head) * kD + 8 * j);
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

constexpr int kProceed = 1;  // fwd_checks: arguments valid and there is work to launch
constexpr int kMaxSplit = 8;
constexpr int kMinTailKeys = 1024;  // a tail tile's key ranges keep at least this many keys

// The tail split of lsv_attn_fwd_tail for n_logical query tiles on `units` workgroup slots
// (units / 8 per XCD). Each XCD owns P = ceil(n_logical / 8) consecutive tiles, as in the plain
// launch (the last XCD fewer when n_logical is not a multiple of 8); the t = P mod (units / 8)
// of them past its last whole round are cut into key ranges when t is at most a quarter of a
// round, into as many ranges as fill the XCD's slots (at most kMaxSplit, and each of at least
// kMinTailKeys keys of a max_seqlen-key segment). n_tail = 8 t. (Measured on MI355X: a round half
// full costs less than a full one -- the idle half lets the busy half clock higher -- and
// cutting it into 2 ranges gained nothing at 4,096 x 56; a round one-sixth full, at 19,394 x
// 14, cut into 6 ranges gained 9%.)
void tail_plan(int64_t n_logical, int32_t max_seqlen, int32_t units, int32_t* n_split, int64_t* n_tail) {
  *n_split = 1;
  *n_tail = 0;
  const int64_t slots = units / 8;
  const int64_t t = ((n_logical + 7) / 8) % slots;
  if (t == 0 || t > slots / 4) return;
  int64_t split = slots / t;
  if (split > kMaxSplit) split = kMaxSplit;
  if (split > max_seqlen / kMinTailKeys) split = max_seqlen / kMinTailKeys;
  if (split < 2) return;
  *n_split = (int32_t)split;
  *n_tail = 8 * t;
}

// The forward's argument checks (before any HIP call): a status to return, or kProceed with the
// number of 256-row query tiles per segment.
int fwd_checks(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads,
               int32_t head_dim, float scale, int64_t* tiles) {
  if (n_seqs < 0 || max_seqlen < 0 || total_tokens < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (n_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return LSV_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return LSV_ERR_ALIGNMENT;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return LSV_ERR_ALIGNMENT;
  if (total_tokens > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  // K/V copies address a segment with 32-bit byte offsets (rows x row stride, 24-bit factors).
  const int64_t row_stride = (int64_t)n_heads * kRowBytes;
  if (row_stride >= (1 << 24) || (int64_t)max_seqlen >= (1 << 24) ||
      (int64_t)max_seqlen * row_stride + kRowBytes > (int64_t)UINT32_MAX)
    return LSV_ERR_UNSUPPORTED;
  *tiles = ((int64_t)max_seqlen + kBQ - 1) / kBQ;
  return kProceed;
}

// lsv_attn_fwd_qnorm's checks beyond the forward's: a status to return, or kProceed with the tiles
// per segment and the Q-side prologue's parameters.
int qnorm_checks(const void* q, const void* k, const void* v, const void* q_weight, const void* cos, const void* sin,
                 int32_t rotary_dim, float eps, const void* o, const float* lse, const int32_t* cu_seqlens,
                 int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                 float scale, int64_t* tiles, QNorm* qn) {
  if (!(eps >= 0.f) || !isfinite(eps)) return LSV_ERR_INVALID_ARG;
  if (rotary_dim < 0 || rotary_dim > kD || rotary_dim % 16 != 0) return LSV_ERR_UNSUPPORTED;
  const int rc = fwd_checks(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                            tiles);
  if (rc != kProceed) return rc;
  if (!q_weight || (rotary_dim > 0 && (!cos || !sin))) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q_weight | (uintptr_t)cos | (uintptr_t)sin) & 15) return LSV_ERR_ALIGNMENT;
  qn->w = (const uint16_t*)q_weight;
  qn->cos = (const uint16_t*)cos;
  qn->sin = (const uint16_t*)sin;
  qn->r = rotary_dim;
  qn->eps = eps;
  return kProceed;
}

}  // namespace

extern "C" {

const char* lsv_status_string(int status) {
  switch (status) {
    case LSV_OK: return "ok";
    case LSV_ERR_INVALID_ARG: return "invalid argument";
    case LSV_ERR_UNSUPPORTED: return "unsupported configuration";
    case LSV_ERR_ALIGNMENT: return "misaligned pointer";
    case LSV_ERR_LAUNCH: return "kernel launch failed";
    case LSV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int lsv_tile_config(int* block_q, int* block_k) {
  if (block_q) *block_q = kBQ;
  if (block_k) *block_k = kBK;
  return LSV_OK;
}

int lsv_device_peak(int device, double* tflops, int* compute_units, int* clock_khz) {
  int cus = 0, khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return LSV_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess) return LSV_ERR_HIP;
  if (tflops) *tflops = (double)cus * (double)khz * 1e3 * 4096.0 / 1e12;
  if (compute_units) *compute_units = cus;
  if (clock_khz) *clock_khz = khz;
  return LSV_OK;
}

int lsv_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                 int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                 float scale, void* stream) {
  int64_t tiles = 0;
  const int rc = fwd_checks(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                            &tiles);
  if (rc != kProceed) return rc;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  const float c = (float)((double)scale * 1.4426950408889634074);
  // The tail kernel with nothing cut: the plain launch's tiles, XCDs, order and arithmetic, and
  // the compiled loop that measured 0.8-1.4% faster than a kernel of the same body with the
  // plain mapping (its LDS operand reads are scheduled further ahead; same-box A/B).
  // The dynamic-LDS limit is a per-function attribute; setting it again is harmless.
  if (hipFuncSetAttribute((const void*)attn_fwd_tail_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_tail_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, cu_seqlens,
                     (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads, total_tokens, c, (int)n_logical, 0, 1,
                     (float*)nullptr, (float*)nullptr);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

int lsv_attn_fwd_qnorm(const void* q, const void* k, const void* v, const void* q_weight, const void* cos,
                       const void* sin, int32_t rotary_dim, float eps, void* o, float* lse,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens,
                       int32_t n_heads, int32_t head_dim, float scale, void* stream) {
  int64_t tiles = 0;
  QNorm qn;
  const int rc = qnorm_checks(q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens, n_seqs, max_seqlen,
                              total_tokens, n_heads, head_dim, scale, &tiles, &qn);
  if (rc != kProceed) return rc;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_qnorm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  const float c = (float)((double)scale * 1.4426950408889634074);
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_qnorm_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, cu_seqlens,
                     (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads, total_tokens, c, (int)n_logical, qn, 0,
                     1, (float*)nullptr, (float*)nullptr);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

int lsv_attn_fwd_qnorm_tail(const void* q, const void* k, const void* v, const void* q_weight, const void* cos,
                            const void* sin, int32_t rotary_dim, float eps, void* o, float* lse,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens,
                            int32_t n_heads, int32_t head_dim, float scale, int32_t compute_units, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  if (compute_units < 8 || compute_units % 8 != 0) return LSV_ERR_INVALID_ARG;
  int64_t tiles = 0;
  QNorm qn;
  const int rc = qnorm_checks(q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens, n_seqs, max_seqlen,
                              total_tokens, n_heads, head_dim, scale, &tiles, &qn);
  if (rc != kProceed) return rc;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  int32_t n_split = 1;
  int64_t n_tail = 0;
  tail_plan(n_logical, max_seqlen, compute_units, &n_split, &n_tail);
  if (n_split == 1)
    return lsv_attn_fwd_qnorm(q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens, n_seqs, max_seqlen,
                              total_tokens, n_heads, head_dim, scale, stream);
  if (!workspace) return LSV_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 15) return LSV_ERR_ALIGNMENT;
  const int64_t pieces = n_tail * n_split;
  if (workspace_bytes < pieces * kBQ * (kD + 1) * (int64_t)sizeof(float)) return LSV_ERR_INVALID_ARG;
  const int64_t grid = (n_logical + 7) / 8 * 8 - n_tail + pieces;  // 8 x (blocks per XCD)
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_qnorm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  float* part_o = (float*)workspace;
  float* part_lse = part_o + pieces * kBQ * kD;
  const float c = (float)((double)scale * 1.4426950408889634074);
  const hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_qnorm_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles,
                     (int)max_seqlen, (int)n_heads, total_tokens, c, (int)n_logical, qn, (int)n_tail, (int)n_split,
                     part_o, part_lse);
  hipLaunchKernelGGL(attn_fwd_tail_combine_kernel, dim3((unsigned)n_tail), dim3(256), 0, st, part_o, part_lse,
                     (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads,
                     total_tokens, (int)n_logical, (int)n_tail, (int)n_split);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

int lsv_attn_fwd_tail_plan(int32_t n_seqs, int32_t max_seqlen, int32_t n_heads, int32_t compute_units,
                           int32_t* n_split, int64_t* n_tail_tiles) {
  if (n_seqs < 0 || max_seqlen < 0 || n_heads < 1 || compute_units < 8 || compute_units % 8 != 0 || !n_split ||
      !n_tail_tiles)
    return LSV_ERR_INVALID_ARG;
  const int64_t tiles = ((int64_t)max_seqlen + kBQ - 1) / kBQ;
  tail_plan(tiles * n_seqs * (int64_t)n_heads, max_seqlen, compute_units, n_split, n_tail_tiles);
  return LSV_OK;
}

int64_t lsv_attn_fwd_tail_workspace_size(int32_t compute_units) {
  if (compute_units < 8 || compute_units % 8 != 0) return -1;
  return (int64_t)compute_units * kBQ * (kD + 1) * (int64_t)sizeof(float);
}

int lsv_attn_fwd_tail(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                      int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                      float scale, int32_t compute_units, void* workspace, int64_t workspace_bytes, void* stream) {
  if (compute_units < 8 || compute_units % 8 != 0) return LSV_ERR_INVALID_ARG;
  int64_t tiles = 0;
  const int rc = fwd_checks(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                            &tiles);
  if (rc != kProceed) return rc;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  int32_t n_split = 1;
  int64_t n_tail = 0;
  tail_plan(n_logical, max_seqlen, compute_units, &n_split, &n_tail);
  if (n_split == 1)
    return lsv_attn_fwd(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                        stream);
  if (!workspace) return LSV_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 15) return LSV_ERR_ALIGNMENT;
  const int64_t pieces = n_tail * n_split;
  if (workspace_bytes < pieces * kBQ * (kD + 1) * (int64_t)sizeof(float)) return LSV_ERR_INVALID_ARG;
  const int64_t grid = (n_logical + 7) / 8 * 8 - n_tail + pieces;  // 8 x (blocks per XCD)
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_tail_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  float* part_o = (float*)workspace;
  float* part_lse = part_o + pieces * kBQ * kD;
  const float c = (float)((double)scale * 1.4426950408889634074);
  const hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_tail_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles,
                     (int)max_seqlen, (int)n_heads, total_tokens, c, (int)n_logical, (int)n_tail, (int)n_split,
                     part_o, part_lse);
  hipLaunchKernelGGL(attn_fwd_tail_combine_kernel, dim3((unsigned)n_tail), dim3(256), 0, st, part_o, part_lse,
                     (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads,
                     total_tokens, (int)n_logical, (int)n_tail, (int)n_split);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

int64_t lsv_attn_fwd_split_workspace_size(int64_t total_tokens, int32_t n_heads, int32_t n_split) {
  if (total_tokens < 0 || n_heads < 1 || n_split < 1 || n_split > kMaxSplit) return -1;
  if (n_split == 1) return 0;
  return (int64_t)n_split * total_tokens * (int64_t)n_heads * (kD + 1) * (int64_t)sizeof(float);
}

int lsv_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens,
                       int32_t n_heads, int32_t head_dim, float scale, int32_t n_split, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (n_split < 1 || n_split > kMaxSplit) return LSV_ERR_INVALID_ARG;
  if (n_split == 1)
    return lsv_attn_fwd(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                        stream);
  int64_t tiles = 0;
  const int rc = fwd_checks(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                            &tiles);
  if (rc != kProceed) return rc;
  if (!workspace) return LSV_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 15) return LSV_ERR_ALIGNMENT;
  if (workspace_bytes < lsv_attn_fwd_split_workspace_size(total_tokens, n_heads, n_split))
    return LSV_ERR_INVALID_ARG;
  const int64_t n_logical = tiles * n_split * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  const int64_t n_logical_c = tiles * n_seqs * (int64_t)n_heads;
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  if (hipFuncSetAttribute((const void*)attn_fwd_split_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsBytes) != hipSuccess)
    return LSV_ERR_HIP;
  float* part_o = (float*)workspace;
  float* part_lse = part_o + (int64_t)n_split * total_tokens * n_heads * kD;
  const float c = (float)((double)scale * 1.4426950408889634074);
  const hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_split_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen,
                     (int)n_heads, total_tokens, c, (int)n_logical, (int)n_split, part_o, part_lse);
  hipLaunchKernelGGL(attn_fwd_combine_kernel, dim3((unsigned)n_logical_c), dim3(256), 0, st, part_o, part_lse,
                     (uint16_t*)o, lse, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen, (int)n_heads,
                     total_tokens, (int)n_logical_c, (int)n_split);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

}  // extern "C"
