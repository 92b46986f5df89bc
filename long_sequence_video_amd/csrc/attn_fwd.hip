// Dense non-causal varlen BF16 attention forward for gfx950 (MI355X), with the C ABI.
//
// The operation is the varlen forward of FastVideo #2049 (diff of
// fastvideo/attention/utils/flash_attn_cute.py): per packed segment, head and query row,
// O = softmax(scale * q K^T) V over the keys of the same segment, plus the natural-log
// LSE, non-causal, one split. TensorRT-LLM PR #21275 (Description) gives the shapes this
// kernel is built for: 19k-104k packed tokens, 56 heads (or one sp=4 rank's 14) x 128.
//
// Design (gfx950, wave64):
//  * One workgroup = 4 waves = 128 query rows of one (segment, head), one wave per SIMD;
//    each wave owns 32 query rows.
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
//    with 16-byte global_load_lds_dwordx4, four tiles ahead of use; one barrier per tile.
//  * Software pipeline per tile t: the 8 MFMAs of O += P(t-1) V(t-1), then the 8 of
//    S(t+1) = Q K(t+1)^T, with the online softmax of S(t) split into small VALU groups
//    placed between them (explicit scheduling barriers hold the order).
//  * Online softmax in the exp2 domain: c = scale * log2(e) is folded into one fp32 FMA
//    per score, p = exp2(s c - m c). The running max is only raised when a row's tile max
//    exceeds it by more than 8 (log2 units), so the O rescale is rare; p stays <= 2^8.
//    P V uses p rounded to bf16 and O is divided by the sum of those same rounded p; the
//    LSE uses the sum of the fp32 p.
//  * LDS rows (256 bytes) are XOR-swizzled in 16-byte chunks so that both the K reads
//    (32 rows, same chunk) and the transposing V reads (4 rows x 32 bytes per 16 lanes)
//    spread over the banks.
//  * Workgroups are remapped so that consecutive tiles of one (head, segment) land on the
//    same XCD (dispatch is round-robin over the 8 XCDs) and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "lsv.h"

namespace {

constexpr int kD = 128;                       // head dim
constexpr int kWaveQ = 32;                    // query rows per wave
constexpr int kWaves = 4;                     // waves per workgroup
constexpr int kBQ = kWaveQ * kWaves;          // query rows per workgroup
constexpr int kBK = 32;                       // keys per tile
constexpr int kSlots = 8;                     // LDS ring slots (K and V each)
constexpr int kAhead = 4;                     // tiles in flight ahead of use
constexpr int kThreads = kWaves * 64;
constexpr int kRowBytes = kD * 2;             // 256
constexpr int kSlotBytes = kBK * kRowBytes;   // 8 KB
constexpr int kRingBytes = kSlots * kSlotBytes;
constexpr int kLdsBytes = 2 * kRingBytes;     // K ring, then V ring: 128 KB
constexpr int kCopies = kSlotBytes / 1024 / kWaves;  // 1 KB copies per wave per tile, for K and for V
constexpr int kOpsPerTile = 2 * kCopies;             // memory instructions per wave per tile
constexpr float kLazyLog2 = 8.0f;             // raise the running max only beyond this (log2 units)
static_assert(kCopies * kWaves * 1024 == kSlotBytes, "tile copies must divide over the waves");
static_assert(kAhead >= 2 && kAhead <= kSlots - 2, "ring too small for the prefetch distance");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte chunk swizzle of an LDS row: chunk c of row r lives at chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Nothing may be scheduled across this point (keeps the hand-placed MFMA / VALU interleave).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// max / sum with the partner lane l ^ 32 (same query, the other 16 keys of each 32).
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

struct Lane {
  int lane, h32, l32;
  unsigned kaddr[8];     // K-ring LDS address of 16-dim step s in slot 0 (slot offsets are immediates)
  unsigned vaddr[4][2];  // V-ring LDS address of d-block db, key half rd in slot 0
};

struct Softmax {
  float m;        // running max (raw score units) of this lane's query
  float l;        // this lane's partial sum of p (fp32) over its 16 of every 32 keys: for LSE
  float lb;       // the same sum of bf16(p), the weights P V uses: normalises O
  float alpha;    // pending O rescale factor
  bool pending;   // wave-uniform: O must be multiplied by alpha before the next P V
};

struct Ctx {
  unsigned lds_base;  // LDS byte address of the dynamic LDS block
  const char* kbase;  // k row `seg_start`, this head
  const char* vbase;
  int64_t row_stride; // bytes between token rows
  int seg_len;
  int wave;
  float c;            // scale * log2(e)
  float lazy;         // kLazyLog2 / c (raw score units)
};

// 16-byte global -> LDS copy per lane: lane i writes LDS bytes [lds + 16 i, lds + 16 i + 16).
// Issued from inline asm so that the compiler does not add its own conservative waits on
// LDS reads; every wait on these copies is explicit (wait_vmcnt) and so is the barrier.
// M0 (the LDS destination base) is written only by these copies in this kernel, so the
// clobber of the reserved register is safe; the compiler's note about it is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* src, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_wave_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that waits for this wave's LDS reads but not for its prefetches.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Copy tile t (32 key rows of one head, rows past the segment repeat its last row) of K
// and V into ring slot t % kSlots. Copy L (1 KB) covers rows 4L .. 4L+3: lane i fills
// physical chunk i % 16 of row 4L + i / 16 with logical chunk (i % 16) ^ swz(row).
__device__ __forceinline__ void load_tile(const Ctx& cx, int t, int lane) {
  const int slot = t & (kSlots - 1);
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int L = cx.wave * kCopies + j;
    const int r = 4 * L + (lane >> 4);
    const int ch = (lane & 15) ^ swz(r);
    int key = t * kBK + r;
    key = key < cx.seg_len ? key : cx.seg_len - 1;
    const int64_t off = (int64_t)key * cx.row_stride + ch * 16;
    const unsigned dst = __builtin_amdgcn_readfirstlane(cx.lds_base + slot * kSlotBytes + L * 1024);
    dma16(cx.kbase + off, dst);
    dma16(cx.vbase + off, dst + kRingBytes);
  }
}

__device__ __forceinline__ bf16x8 lds_k(unsigned addr) { return *(lds_bf16x8*)(uintptr_t)addr; }

__device__ __forceinline__ bf16x8 lds_v_tr(unsigned a0, unsigned a1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
  u32x4 u;
  u[0] = __builtin_bit_cast(u32x2, a)[0];
  u[1] = __builtin_bit_cast(u32x2, a)[1];
  u[2] = __builtin_bit_cast(u32x2, b)[0];
  u[3] = __builtin_bit_cast(u32x2, b)[1];
  return __builtin_bit_cast(bf16x8, u);
}

// V operand i (key chunk kc = i / 4, d-block db = i % 4) of the tile in ring byte offset `slot`.
__device__ __forceinline__ bf16x8 v_operand(const Lane& ln, unsigned slot, int i) {
  const int kc = i >> 2, db = i & 3;
  return lds_v_tr(ln.vaddr[db][0] + slot + kc * 16 * kRowBytes, ln.vaddr[db][1] + slot + kc * 16 * kRowBytes);
}

// S^T (32 keys x 32 queries) = K(slot) Q^T: 8 MFMAs over the 128 dims (used outside the
// steady state).
__device__ __forceinline__ f32x16 qk_tile(unsigned slot, const bf16x8 (&qr)[8], const Lane& ln) {
  f32x16 S = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) S = mfma(lds_k(ln.kaddr[s] + slot), qr[s], S);
  return S;
}

// O^T (128 dims x 32 queries) += V(slot)^T P^T: 2 key chunks of 16 x 4 d-blocks of 32.
__device__ __forceinline__ void pv_tile(f32x16 (&O)[4], unsigned slot, const bf16x8 (&P)[2], const Lane& ln) {
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i & 3] = mfma(v_operand(ln, slot, i), P[i >> 2], O[i & 3]);
}

// Online softmax, part 1: row max of S, lazy max update, pending rescale factor.
// Branch-free: when some row's tile max exceeds its running max by more than the lazy
// margin, every row of the wave takes m = max(m, tile max) and the pending O rescale
// factor is multiplied by exp2((m_old - m_new) c) (1 for rows whose max did not move).
// Returns -m c (the FMA addend of part 2) and scales the running sum.
__device__ __forceinline__ float softmax_max(const f32x16& S, Softmax& st, const Ctx& cx) {
  float mx = fmaxf(fmaxf(S[0], S[1]), S[2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) mx = fmaxf(fmaxf(mx, S[v]), S[v + 1]);
  mx = fmaxf(mx, S[15]);
  mx = pair_max(mx);
  const bool raise = __builtin_amdgcn_ballot_w64(mx > st.m + cx.lazy) != 0;  // wave-uniform
  const float mnew = raise ? fmaxf(st.m, mx) : st.m;
  const float a = __builtin_amdgcn_exp2f((st.m - mnew) * cx.c);
  st.alpha = raise ? st.alpha * a : st.alpha;
  st.pending = st.pending || raise;
  st.m = mnew;
  st.l *= a;
  st.lb *= a;
  return -mnew * cx.c;
}

// Online softmax, part 2 on scores 2j, 2j+1: p = exp2(s c - m c) -> bf16 pair. Two row sums:
// the fp32 p (for the LSE; a sum of rounded p would move it by up to ~2^-9) and the bf16 p
// (v_dot2_f32_bf16; O is divided by the sum of exactly the weights that multiplied V).
__device__ __forceinline__ void softmax_pair(const f32x16& S, u32x4 (&P)[2], Softmax& st, const Ctx& cx, float nmc,
                                             int j) {
  const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * j], cx.c, nmc));
  const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * j + 1], cx.c, nmc));
  st.l += e0;
  st.l += e1;
  bf16x2 pp, one;
  pp[0] = (__bf16)e0;
  pp[1] = (__bf16)e1;
  one[0] = (__bf16)1.0f;
  one[1] = (__bf16)1.0f;
  st.lb = __builtin_amdgcn_fdot2_f32_bf16(pp, one, st.lb, false);
  P[j >> 2][j & 3] = __builtin_bit_cast(unsigned, pp);
}

// Whole-tile softmax (outside the steady state). MASK: keys at and past `valid` are outside
// the segment; element v holds key 8 (v / 4) + 4 h32 + v % 4.
template <bool MASK>
__device__ __forceinline__ void softmax_tile(f32x16 S, bf16x8 (&P)[2], Softmax& st, const Ctx& cx, int valid,
                                             const Lane& ln) {
  if constexpr (MASK) {
    const int lim = valid - 4 * ln.h32;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (8 * (v >> 2) + (v & 3) >= lim) S[v] = -INFINITY;
  }
  const float nmc = softmax_max(S, st, cx);
  u32x4 p[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) softmax_pair(S, p, st, cx, nmc, j);
  P[0] = __builtin_bit_cast(bf16x8, p[0]);
  P[1] = __builtin_bit_cast(bf16x8, p[1]);
}

__device__ __forceinline__ void apply_rescale(f32x16 (&O)[4], Softmax& st) {
  if (st.pending) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][v] *= st.alpha;
    st.pending = false;
    st.alpha = 1.f;
  }
}

// Steady-state tile t (1 <= t <= n_kt - 2, t % kSlots == U):
//   O += P(t-1) V(t-1) (8 MFMAs), then S(t+1) = Q K(t+1)^T (8 MFMAs); the softmax of S(t)
//   (row max, then 8 pairs of exp2) runs in small VALU groups between them; then the copy
//   of tile t + kAhead is issued, tile t+2 is waited for, and the workgroup synchronises.
template <int U>
__device__ __forceinline__ void step(const Ctx& cx, int t, f32x16 (&O)[4], const f32x16& Scur, f32x16& Snext,
                                     const bf16x8 (&Pprev)[2], bf16x8 (&Pcur)[2], Softmax& st,
                                     const bf16x8 (&qr)[8], const Lane& ln) {
  constexpr unsigned vslot = ((U + kSlots - 1) % kSlots) * kSlotBytes;
  constexpr unsigned kslot = ((U + 1) % kSlots) * kSlotBytes;
  apply_rescale(O, st);
  // LDS operands are read in halves, a few MFMAs ahead of use, to bound register use.
  bf16x8 va[8], ka[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) va[i] = v_operand(ln, vslot, i);
  sched_fence();
  // P V MFMA 0 with the row max and lazy update of S(t).
  O[0] = mfma(va[0], Pprev[0], O[0]);
  const float nmc = softmax_max(Scur, st, cx);
  sched_fence();
#pragma unroll
  for (int i = 4; i < 8; ++i) va[i] = v_operand(ln, vslot, i);
  O[1] = mfma(va[1], Pprev[0], O[1]);
  sched_fence();
  u32x4 p[2];
  // P V MFMAs 2..7, one exp2 pair each; K operands of S(t+1) read in between.
#pragma unroll
  for (int i = 2; i < 8; ++i) {
    if (i == 4) {
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = lds_k(ln.kaddr[s] + kslot);
    }
    if (i == 6) {
#pragma unroll
      for (int s = 4; s < 8; ++s) ka[s] = lds_k(ln.kaddr[s] + kslot);
    }
    O[i & 3] = mfma(va[i], Pprev[i >> 2], O[i & 3]);
    softmax_pair(Scur, p, st, cx, nmc, i - 2);
    sched_fence();
  }
  // Q K^T MFMAs, the last two exp2 pairs.
  f32x16 S = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    S = mfma(ka[s], qr[s], S);
    if (s < 2) softmax_pair(Scur, p, st, cx, nmc, 6 + s);
    sched_fence();
  }
  Snext = S;
  Pcur[0] = __builtin_bit_cast(bf16x8, p[0]);
  Pcur[1] = __builtin_bit_cast(bf16x8, p[1]);
  // P(t) and the row sum must be complete here (they must not sink into the next tile).
  asm volatile("" : "+v"(Pcur[0]), "+v"(Pcur[1]), "+v"(st.l), "+v"(st.lb));
  load_tile(cx, t + kAhead, ln.lane);
  wait_vmcnt<kOpsPerTile * (kAhead - 2)>();
  barrier_lds();
}

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                uint16_t* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ cu_seqlens,
                int n_seqs, int tiles_per_seq, int n_heads, int64_t total_tokens, float c, float lazy,
                int n_logical) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];

  // XCD-aware order: hardware dispatches block b to XCD b % 8; give each XCD a contiguous
  // range of logical tiles (head-major, then segment, then query tile).
  const int per_xcd = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= n_logical) return;
  const int qt = logical % tiles_per_seq;
  const int hs = logical / tiles_per_seq;
  const int seg = hs % n_seqs;
  const int head = hs / n_seqs;
  const int seg_start = cu_seqlens[seg];
  const int seg_end = cu_seqlens[seg + 1];
  if (seg_start < 0 || seg_end < seg_start || (int64_t)seg_end > total_tokens) return;
  const int seg_len = seg_end - seg_start;
  const int q0 = qt * kBQ;
  if (q0 >= seg_len) return;

  const int tid = threadIdx.x;
  Ctx cx;
  cx.lds_base = (unsigned)(uintptr_t)(lds_char*)smem_generic;
  cx.wave = tid >> 6;
  cx.row_stride = (int64_t)n_heads * kRowBytes;
  cx.kbase = (const char*)k + ((int64_t)seg_start * n_heads + head) * kRowBytes;
  cx.vbase = (const char*)v + ((int64_t)seg_start * n_heads + head) * kRowBytes;
  cx.seg_len = seg_len;
  cx.c = c;
  cx.lazy = lazy;
  const int n_kt = (seg_len + kBK - 1) / kBK;

  Lane ln;
  ln.lane = tid & 63;
  ln.h32 = ln.lane >> 5;
  ln.l32 = ln.lane & 31;
  {
    const int sw = swz(ln.l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) ln.kaddr[s] = cx.lds_base + ln.l32 * kRowBytes + ((((2 * s) | ln.h32) ^ sw) << 4);
    const int i = ln.lane & 15, g2 = (ln.lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int row = 8 * rd + 4 * ln.h32 + (i >> 2);
        const int chunk = 4 * db + 2 * g2 + ((i & 3) >> 1);
        ln.vaddr[db][rd] = cx.lds_base + kRingBytes + row * kRowBytes + ((chunk ^ swz(row)) << 4) + 8 * (i & 1);
      }
  }

  // Q^T operand: lane holds q[row][16 s + 8 h32 .. +7] for s = 0..7.
  bf16x8 qr[8];
  {
    int row = q0 + cx.wave * kWaveQ + ln.l32;
    row = row < seg_len ? row : seg_len - 1;
    const char* qrow = (const char*)q + ((int64_t)(seg_start + row) * n_heads + head) * kRowBytes + ln.h32 * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) qr[s] = *(const bf16x8*)(qrow + s * 32);
  }

  // Prologue: tiles 0 .. kAhead-1 in flight (tiles past the segment repeat its last row);
  // wait for tiles 0 and 1.
#pragma unroll
  for (int t = 0; t < kAhead; ++t) load_tile(cx, t, ln.lane);
  wait_vmcnt<kOpsPerTile * (kAhead - 2)>();
  barrier_lds();

  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};
  f32x16 SA, SB;
  bf16x8 PA[2], PB[2];
  Softmax st{-INFINITY, 0.f, 0.f, 1.f, false};
  SA = qk_tile(0, qr, ln);

  // Tile 0: no P V yet.
  if (n_kt == 1) {
    softmax_tile<true>(SA, PA, st, cx, seg_len, ln);
  } else {
    softmax_tile<false>(SA, PA, st, cx, kBK, ln);
    SB = qk_tile(1 * kSlotBytes, qr, ln);
    load_tile(cx, kAhead, ln.lane);
    wait_vmcnt<kOpsPerTile * (kAhead - 2)>();
    barrier_lds();
  }

  // Tiles 1 .. n_kt-2, two per iteration (odd t, then even t + 1). S(t) is in SA for even
  // t, SB for odd t; P(t) likewise in PA / PB.
  int t = 1;
  for (; t + 1 <= n_kt - 2; t += 2) {
    switch (t & (kSlots - 1)) {
      case 1: step<1>(cx, t, O, SB, SA, PA, PB, st, qr, ln); step<2>(cx, t + 1, O, SA, SB, PB, PA, st, qr, ln); break;
      case 3: step<3>(cx, t, O, SB, SA, PA, PB, st, qr, ln); step<4>(cx, t + 1, O, SA, SB, PB, PA, st, qr, ln); break;
      case 5: step<5>(cx, t, O, SB, SA, PA, PB, st, qr, ln); step<6>(cx, t + 1, O, SA, SB, PB, PA, st, qr, ln); break;
      default: step<7>(cx, t, O, SB, SA, PA, PB, st, qr, ln); step<0>(cx, t + 1, O, SA, SB, PB, PA, st, qr, ln); break;
    }
  }
  if (t <= n_kt - 2) {
    switch (t & (kSlots - 1)) {
      case 1: step<1>(cx, t, O, SB, SA, PA, PB, st, qr, ln); break;
      case 3: step<3>(cx, t, O, SB, SA, PA, PB, st, qr, ln); break;
      case 5: step<5>(cx, t, O, SB, SA, PA, PB, st, qr, ln); break;
      default: step<7>(cx, t, O, SB, SA, PA, PB, st, qr, ln); break;
    }
  }

  // Last tile (n_kt >= 2): P V of tile n_kt-2, masked softmax of tile n_kt-1.
  const int tl = n_kt - 1;
  if (tl >= 1) {
    apply_rescale(O, st);
    const unsigned vprev = ((tl - 1) & (kSlots - 1)) * kSlotBytes;
    const int valid = seg_len - tl * kBK;
    if (tl & 1) {
      pv_tile(O, vprev, PA, ln);
      softmax_tile<true>(SB, PB, st, cx, valid, ln);
    } else {
      pv_tile(O, vprev, PB, ln);
      softmax_tile<true>(SA, PA, st, cx, valid, ln);
    }
  }
  // P V of the last tile.
  apply_rescale(O, st);
  {
    const unsigned vlast = (tl & (kSlots - 1)) * kSlotBytes;
    if (tl & 1) pv_tile(O, vlast, PB, ln);
    else pv_tile(O, vlast, PA, ln);
  }
  // No copy may still be writing this workgroup's LDS when it exits.
  wait_vmcnt<0>();

  // Epilogue: O / lb -> bf16, LSE = (m c + log2 l) ln 2.
  const float l = pair_sum(st.l);
  const float lb = pair_sum(st.lb);
  const int row = q0 + cx.wave * kWaveQ + ln.l32;
  if (row < seg_len) {
    const int64_t tok = (int64_t)seg_start + row;
    uint16_t* orow = o + (tok * n_heads + head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x2 lo, hi;
        lo[0] = (__bf16)(O[db][4 * g + 0] / lb);
        lo[1] = (__bf16)(O[db][4 * g + 1] / lb);
        hi[0] = (__bf16)(O[db][4 * g + 2] / lb);
        hi[1] = (__bf16)(O[db][4 * g + 3] / lb);
        u32x2 pk;
        pk[0] = __builtin_bit_cast(unsigned, lo);
        pk[1] = __builtin_bit_cast(unsigned, hi);
        *(u32x2*)(orow + 32 * db + 8 * g + 4 * ln.h32) = pk;
      }
    if (ln.h32 == 0) lse[(int64_t)head * total_tokens + tok] = (st.m * c + __log2f(l)) * 0.69314718055994530942f;
  }
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
  if (n_seqs < 0 || max_seqlen < 0 || total_tokens < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (n_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return LSV_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return LSV_ERR_ALIGNMENT;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return LSV_ERR_ALIGNMENT;
  if (total_tokens > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  const int64_t tiles = ((int64_t)max_seqlen + kBQ - 1) / kBQ;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  if (grid > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  // The dynamic-LDS limit is a per-function attribute; setting it again is harmless.
  if (hipFuncSetAttribute((const void*)attn_fwd_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) !=
      hipSuccess)
    return LSV_ERR_HIP;
  const float c = (float)((double)scale * 1.4426950408889634074);
  const float lazy = kLazyLog2 / c;
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, cu_seqlens,
                     (int)n_seqs, (int)tiles, (int)n_heads, total_tokens, c, lazy, (int)n_logical);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

}  // extern "C"
