// Backward of the dense non-causal varlen BF16 attention for gfx950 (MI355X), with the C ABI.
//
// The operation is the varlen backward op of FastVideo #2049 (diff of
// fastvideo/attention/utils/flash_attn_cute.py: it takes q, k, v, out, dout, lse, the softmax
// scale, causal=False and the forward's cu_seqlens / max_seqlen, and returns dq, dk, dv shaped
// like q, k, v). Per segment, head, query i and key j, with P_ij = exp(scale q_i.k_j - LSE_i):
//   D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . v_j - D_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i.
//
// Design (gfx950, wave64), two kernels on the caller's stream (prep, then the dK/dV and dQ
// passes in one launch), no atomics (deterministic):
//  * prep: -LSE / scale and -D per (head, token) into the workspace (16 lanes per row, like
//    the other row-streaming passes). In raw score units, P = exp2(log2(e) scale (s - LSE /
//    scale)), so the dK/dV pass starts its S accumulator at -LSE / scale and its dP
//    accumulator at -D: the products come out as s - LSE / scale and dP - D, and each
//    element then costs one multiply and one exp2 for P and one multiply for dS.
//  * dK/dV: one workgroup = 8 waves = 256 keys of one (segment, head); each wave owns 32 keys
//    with K and V held in registers as MFMA B operands. Query tiles of 32 rows stream through
//    a 4-slot LDS ring, each stored twice: in the row layout (A operand of S = Q K^T and
//    dP = dO V^T) and in the transposed-read layout (A operand of dK^T += Q^T dS and
//    dV^T += dO^T P), plus the tile's -LSE / scale and -D. The S and dP accumulators give a
//    lane one key and 16 queries; P and dS converted to bf16 are the B operands of the two
//    accumulating products as they are.
//  * dQ: one workgroup = 256 queries; K and V tiles of 32 keys stream through the ring (K in
//    both layouts, V in the row layout); S^T = K Q^T and dP^T = V dO^T give a lane one query
//    and 16 keys, dS^T in bf16 is the B operand of dQ^T += K^T dS^T.
//  * The two passes are independent, so they share one launch, dQ blocks after dK/dV blocks:
//    a launch with few tiles then has one partly idle last round instead of two.
//  * Copies are 16-byte global -> LDS transfers issued three tiles ahead; the last, partial
//    tile of a segment is read shifted back to end at the segment end and its re-read rows
//    are masked (segments shorter than 32 rows repeat their last row instead).
//  * Each tile is one fixed sequence of MFMAs (24 in dQ, 32 in dK/dV) whose LDS operands are
//    read two MFMAs ahead, with the vector work placed between them; scheduling barriers hold
//    the order. The register operands (Q, dO in dQ; K, V in dK/dV) are waited for before the
//    first tile copy, so no wait inside the loop counts the copies in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <mutex>

#include "lsv.h"
#include "tile_ops.h"

namespace {

using namespace lsv_tiles;

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockRows = kWaves * 32;   // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBT = kTileRows;            // rows per streamed tile
constexpr int kSlots = 4;                 // ring slots
constexpr int kAhead = 3;                 // tiles in flight ahead of use
constexpr int kRing = kSlots * kTileBytes;  // one region of the ring: 32 KB
static_assert(kAhead <= kSlots - 1, "a slot is reloaded only after every wave has left it");

// dQ kernel LDS: K rows | V rows | K transposed-read, one 32 KB ring region each.
constexpr int kDqLds = 3 * kRing;
constexpr int kDqOps = 3;                 // copies per wave per tile
// dK/dV kernel LDS: Q rows | dO rows | Q transposed | dO transposed | stats.
constexpr int kStatBytes = 2 * kBT * 4;   // 32 floats of -LSE / scale, 32 of -D
constexpr int kDkvLds = 4 * kRing + kSlots * kStatBytes;
constexpr int kDkvOps = 5;

// 4-byte global -> LDS copy per lane: lane i writes LDS bytes [lds + 4 i, lds + 4 i + 4).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(unsigned voff, const char* base, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, %2" ::"v"(voff), "s"(lds_wave_base), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ float lo_f(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// Element v of an accumulator holds row 8 (v / 4) + 4 h32 + v % 4 of its 32-row tile. Rows
// outside [lo, hi) get -inf, in place.
__device__ __forceinline__ void mask_rows(f32x16& S, int lo, int hi, int h32) {
  const int a = lo - 4 * h32, b = hi - 4 * h32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 8 * (v >> 2) + (v & 3);
    S[v] = (r >= a && r < b) ? S[v] : -INFINITY;
  }
}

__device__ __forceinline__ void pack_pair(u32x4 (&P)[2], int j, float a, float b) {
  bf16x2 pp;
  pp[0] = (__bf16)a;  // round to nearest even
  pp[1] = (__bf16)b;
  P[j >> 2][j & 3] = __builtin_bit_cast(unsigned, pp);
}

// Block b of a pass -> (head, segment, 256-row tile), XCD-aware: hardware dispatches block b
// to XCD b % 8 (a pass starts at a multiple of 8); each XCD gets a contiguous range of
// per_xcd logical tiles (head-major, then segment).
struct Work {
  int head, seg_start, seg_len, r0;
  bool ok;
};
__device__ __forceinline__ Work map_block(int b, int per_xcd, const int32_t* cu_seqlens, int n_seqs,
                                          int tiles_per_seq, int max_seqlen, int64_t total_tokens, int n_logical) {
  Work w;
  const int logical = (b & 7) * per_xcd + (b >> 3);
  w.ok = false;
  if (logical >= n_logical) return w;
  const int rt = logical % tiles_per_seq;
  const int hs = logical / tiles_per_seq;
  const int seg = hs % n_seqs;
  w.head = hs / n_seqs;
  w.seg_start = cu_seqlens[seg];
  const int seg_end = cu_seqlens[seg + 1];
  if (w.seg_start < 0 || seg_end < w.seg_start || (int64_t)seg_end > total_tokens) return w;
  w.seg_len = seg_end - w.seg_start;
  if (w.seg_len > max_seqlen) return w;  // breaks the contract; 32-bit copy offsets assume <= max_seqlen
  w.r0 = rt * kBlockRows;
  w.ok = w.r0 < w.seg_len;
  return w;
}

// Copy geometry shared by the streaming kernels: the tile's first row, uniform.
__device__ __forceinline__ int tile_start(int t, int seg_len) { return min(t * kBT, seg_len - kBT); }

// Masks the rows of the last of n_t tiles that are not this segment's own: a shifted tile
// repeats its first 32 n_t - seg_len rows from the tile before, a single short tile (a
// segment under 32 rows) repeats the segment's last row past seg_len.
__device__ __forceinline__ void mask_last_tile(f32x16& S, int seg_len, int n_t, int h32) {
  const int lo = seg_len >= kBT ? kBT * n_t - seg_len : 0;
  const int hi = seg_len >= kBT ? kBT : seg_len;
  mask_rows(S, lo, hi, h32);
}

// ---------------------------------------------------------------------------- prep

__global__ void __launch_bounds__(256)
bwd_prep_kernel(const u32x4* __restrict__ o, const u32x4* __restrict__ dout, const float* __restrict__ lse,
                float* __restrict__ ws_nl, float* __restrict__ ws_d, unsigned n_rows, unsigned n_heads,
                int64_t total_tokens, float inv_scale) {
  const int j = threadIdx.x & 15;
  const unsigned stride = gridDim.x * 16;
  for (unsigned row = blockIdx.x * 16 + (threadIdx.x >> 4); row < n_rows; row += stride) {
    const int64_t idx = (int64_t)row * (kD / 8) + j;
    const u32x4 a = o[idx], b = dout[idx];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(lo_f(a[i]), lo_f(b[i]), acc);
      acc = __builtin_fmaf(hi_f(a[i]), hi_f(b[i]), acc);
    }
    acc += __shfl_xor(acc, 8, 16);
    acc += __shfl_xor(acc, 4, 16);
    acc += __shfl_xor(acc, 2, 16);
    acc += __shfl_xor(acc, 1, 16);
    if (j == 0) {
      const unsigned t = row / n_heads, h = row % n_heads;
      const int64_t s = (int64_t)h * total_tokens + t;
      ws_d[s] = -acc;                   // -D
      ws_nl[s] = -lse[s] * inv_scale;  // -LSE / scale
    }
  }
}

// ---------------------------------------------------------------------------- dQ

struct DqCtx {
  const char* kbase;    // k row seg_start, this head (uniform)
  const char* vbase;
  unsigned row_stride;
  int seg_len;
  unsigned lds_copy;    // this wave's 1 KB block in slot 0 of ring region 0 (uniform)
  int rrow, trow;       // copy rows (row layout, transposed layout)
  unsigned roff, toff;  // byte offsets of the copied chunk inside the row
  unsigned rconst, tconst;  // rrow * row_stride + roff, trow * row_stride + toff
};

// Segments of 32 keys or more: tile t is rows tile_start(t) .. +31 (uniform offset).
__device__ __forceinline__ void dq_load(const DqCtx& cx, int t) {
  const unsigned lds = cx.lds_copy + (unsigned)(t & (kSlots - 1)) * kTileBytes;
  const unsigned off = (unsigned)tile_start(t, cx.seg_len) * cx.row_stride;
  dma16(cx.rconst, cx.kbase + off, lds);
  dma16(cx.rconst, cx.vbase + off, lds + kRing);
  dma16(cx.tconst, cx.kbase + off, lds + 2 * kRing);
}

// A single tile shorter than 32 keys (slot 0): rows past the segment repeat its last row.
__device__ __forceinline__ void dq_load_short(const DqCtx& cx) {
  const unsigned last = (unsigned)cx.seg_len - 1;
  const unsigned r = min((unsigned)cx.rrow, last), tr = min((unsigned)cx.trow, last);
  dma16(__umul24(r, cx.row_stride) + cx.roff, cx.kbase, cx.lds_copy);
  dma16(__umul24(r, cx.row_stride) + cx.roff, cx.vbase, cx.lds_copy + kRing);
  dma16(__umul24(tr, cx.row_stride) + cx.toff, cx.kbase, cx.lds_copy + 2 * kRing);
}

struct DqLane {
  int lane, h32, l32;
  unsigned raddr[8];  // row-layout read address of 16-dim step s (region 0, slot 0)
  unsigned taddr;     // transposed-read lane base (region 2, slot 0)
};

template <int U>
__device__ __forceinline__ void dq_step(const DqCtx& cx, const DqLane& ln, int t, int n_t, const bf16x8 (&qr)[8],
                                        const bf16x8 (&dor)[8], float nl, const f32x16& dinit, float c,
                                        f32x16 (&acc)[4]) {
  constexpr unsigned slot = U * kTileBytes;
  wait_vmcnt<kDqOps * (kAhead - 1)>();
  barrier_lds();
  if (n_t > 1) dq_load(cx, t + kAhead);  // a single-tile segment needs no prefetch
  // One sequence of 24 MFMAs: n = 0..7 S^T (K rows), 8..15 the dP^T chain (V rows, started at
  // -D) with the exp2 work of P between its MFMAs, 16..23 dQ^T += K^T dS^T (K transposed).
  // Every LDS operand is read two MFMAs ahead of its use; scheduling barriers hold the order.
  bf16x8 op[24];
  auto read = [&](int n) {
    if (n < 8) op[n] = lds_row(ln.raddr[n] + slot);
    else if (n < 16) op[n] = lds_row(ln.raddr[n - 8] + slot + kRing);
    else op[n] = tr_operand(ln.taddr, slot, n - 16);
  };
  read(0);
  read(1);
  sched_fence();
  f32x16 S = {}, dP = dinit;
  float p[16];
  u32x4 ds[2];
  bf16x8 dsb[2];
#pragma unroll
  for (int n = 0; n < 24; ++n) {
    if (n + 2 < 24) read(n + 2);
    sched_fence();
    if (n < 8) {
      S = mfma(op[n], qr[n], S);
      if (n == 7 && t == n_t - 1) {
        sched_fence();
        mask_last_tile(S, cx.seg_len, n_t, ln.h32);
      }
    } else if (n < 16) {
      const int s = n - 8;
      dP = mfma(op[n], dor[s], dP);
      sched_fence();
      p[2 * s] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * s], c, nl));
      p[2 * s + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * s + 1], c, nl));
    } else {
      const int i = n - 16;
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) pack_pair(ds, j, p[2 * j] * dP[2 * j], p[2 * j + 1] * dP[2 * j + 1]);
        dsb[0] = __builtin_bit_cast(bf16x8, ds[0]);
      }
      acc[i & 3] = mfma(op[n], dsb[i >> 2], acc[i & 3]);
      sched_fence();
      if (i < 4) {
        const int j = 4 + i;
        pack_pair(ds, j, p[2 * j] * dP[2 * j], p[2 * j + 1] * dP[2 * j + 1]);
        if (i == 3) dsb[1] = __builtin_bit_cast(bf16x8, ds[1]);
      }
    }
    sched_fence();
  }
}

// dQ for the 256 queries of work item w.
__device__ __forceinline__ void dq_body(const Work& w, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                        const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                        const float* __restrict__ ws_nl, const float* __restrict__ ws_d,
                                        uint16_t* __restrict__ dq, int n_heads, int64_t total_tokens, float c,
                                        float scale) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned lds_base = (unsigned)(uintptr_t)(lds_char*)smem_generic;

  DqCtx cx;
  cx.row_stride = (unsigned)n_heads * kRowBytes;
  cx.kbase = (const char*)k + ((int64_t)w.seg_start * n_heads + w.head) * kRowBytes;
  cx.vbase = (const char*)v + ((int64_t)w.seg_start * n_heads + w.head) * kRowBytes;
  cx.seg_len = w.seg_len;
  cx.lds_copy = lds_base + wave * 1024;
  row_copy_lane(wave, tid & 63, cx.rrow, cx.roff);
  tr_copy_lane(wave, tid & 63, cx.trow, cx.toff);
  cx.rconst = (unsigned)cx.rrow * cx.row_stride + cx.roff;
  cx.tconst = (unsigned)cx.trow * cx.row_stride + cx.toff;

  DqLane ln;
  ln.lane = tid & 63;
  ln.h32 = ln.lane >> 5;
  ln.l32 = ln.lane & 31;
#pragma unroll
  for (int s = 0; s < 8; ++s) ln.raddr[s] = row_read_addr(lds_base, ln.l32, ln.h32, s);
  ln.taddr = tr_read_base(lds_base + 2 * kRing, ln.lane);

  // This lane's query: Q^T and dO^T operands (q[row][16 s + 8 h32 .. +7]), its -LSE log2 e, D.
  int row = w.r0 + wave * 32 + ln.l32;
  const bool live = row < w.seg_len;
  row = live ? row : w.seg_len - 1;
  const int64_t tok = (int64_t)w.seg_start + row;
  bf16x8 qr[8], dor[8];
  {
    const int64_t off = (tok * n_heads + w.head) * kD + ln.h32 * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qr[s] = *(const bf16x8*)(q + off + 16 * s);
      dor[s] = *(const bf16x8*)(dout + off + 16 * s);
    }
  }
  // As in the dK/dV kernel: wait for these before any tile copy is issued.
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(qr[s]), "v"(dor[s]));
  const float nl = c * ws_nl[(int64_t)w.head * total_tokens + tok];  // -LSE log2(e)
  f32x16 dinit;  // -D in every element: the starting value of each tile's dP^T
  {
    const float nd = ws_d[(int64_t)w.head * total_tokens + tok];
#pragma unroll
    for (int e = 0; e < 16; ++e) dinit[e] = nd;
  }

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  const int n_t = (w.seg_len + kBT - 1) / kBT;
  if (w.seg_len >= kBT) {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) dq_load(cx, t);
  } else {
    dq_load_short(cx);
    // One tile's copies are fewer than the steps' waits leave in flight, so those waits would
    // not cover them: wait for them here (the step's barrier then publishes every wave's part).
    wait_vmcnt<0>();
  }
  for (int t = 0; t < n_t; t += kSlots) {
    dq_step<0>(cx, ln, t, n_t, qr, dor, nl, dinit, c, acc);
    if (t + 1 < n_t) dq_step<1>(cx, ln, t + 1, n_t, qr, dor, nl, dinit, c, acc);
    if (t + 2 < n_t) dq_step<2>(cx, ln, t + 2, n_t, qr, dor, nl, dinit, c, acc);
    if (t + 3 < n_t) dq_step<3>(cx, ln, t + 3, n_t, qr, dor, nl, dinit, c, acc);
  }
  wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS when it exits

  if (live) {
    uint16_t* orow = dq + (tok * n_heads + w.head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 tmp[2];
        pack_pair(tmp, 0, acc[db][4 * g + 0] * scale, acc[db][4 * g + 1] * scale);
        pack_pair(tmp, 1, acc[db][4 * g + 2] * scale, acc[db][4 * g + 3] * scale);
        u32x2 pk;
        pk[0] = tmp[0][0];
        pk[1] = tmp[0][1];
        *(u32x2*)(orow + 32 * db + 8 * g + 4 * ln.h32) = pk;
      }
  }
}

// ---------------------------------------------------------------------------- dK / dV

struct KvCtx {
  const char* qbase;    // q row seg_start, this head (uniform)
  const char* dobase;
  const char* nlbase;   // ws_nl[head][seg_start] (uniform)
  const char* dbase;
  unsigned row_stride;
  int seg_len;
  unsigned lds_copy;    // this wave's 1 KB block in slot 0 of ring region 0
  unsigned lds_stat;    // this wave's 32-byte block in stats slot 0
  const char* statbase; // nlbase or dbase, by wave, plus this wave's 8 floats (uniform)
  int rrow, trow;
  unsigned roff, toff, rconst, tconst;
  int stat_row;         // row of this lane's stats float
};

// Segments of 32 queries or more: tile t is rows tile_start(t) .. +31 (uniform offset).
__device__ __forceinline__ void kv_load(const KvCtx& cx, int t, int lane) {
  const unsigned lds = cx.lds_copy + (unsigned)(t & (kSlots - 1)) * kTileBytes;
  const unsigned lstat = cx.lds_stat + (unsigned)(t & (kSlots - 1)) * kStatBytes;
  const int start = tile_start(t, cx.seg_len);
  const unsigned off = (unsigned)start * cx.row_stride;
  dma16(cx.rconst, cx.qbase + off, lds);
  dma16(cx.rconst, cx.dobase + off, lds + kRing);
  dma16(cx.tconst, cx.qbase + off, lds + 2 * kRing);
  dma16(cx.tconst, cx.dobase + off, lds + 3 * kRing);
  // One stats copy per wave, lanes 0..7. The lane offset is recomputed here (lane id from
  // v_mbcnt, in a volatile statement the compiler cannot hoist): a register held across the
  // loop would be spilled, and its reload would make the compiler drain every prefetch.
  unsigned lid;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0" : "=v"(lid));
  if (lane < 8) dma4(lid * 4u, cx.statbase + 4 * start, lstat);
}

// A single tile shorter than 32 queries (slot 0): rows past the segment repeat its last row.
__device__ __forceinline__ void kv_load_short(const KvCtx& cx, int lane, int wave) {
  const unsigned last = (unsigned)cx.seg_len - 1;
  const unsigned r = min((unsigned)cx.rrow, last), tr = min((unsigned)cx.trow, last);
  dma16(__umul24(r, cx.row_stride) + cx.roff, cx.qbase, cx.lds_copy);
  dma16(__umul24(r, cx.row_stride) + cx.roff, cx.dobase, cx.lds_copy + kRing);
  dma16(__umul24(tr, cx.row_stride) + cx.toff, cx.qbase, cx.lds_copy + 2 * kRing);
  dma16(__umul24(tr, cx.row_stride) + cx.toff, cx.dobase, cx.lds_copy + 3 * kRing);
  if (lane < 8) dma4(4u * min((unsigned)cx.stat_row, last), cx.statbase - 32 * (wave & 3), cx.lds_stat);
}

struct KvLane {
  int lane, h32, l32;
  unsigned raddr0;    // row-layout read address of 16-dim step 0 (region 0, slot 0); step s is
                      // raddr0 ^ (s << 5): the step only flips chunk bits 1..3 of the swizzle
  unsigned qtaddr;    // transposed-read lane base, region 2 (Q); region 3 (dO) is + kRing
  unsigned staddr;    // this lane's stats: float 8 a + 4 h32 of the tile, a = 0..3 (slot 0)
};


template <int U>
__device__ __forceinline__ void kv_step(const KvCtx& cx, const KvLane& ln, int t, int n_t, const bf16x8 (&kr)[8],
                                        const bf16x8 (&vr)[8], float c, f32x16 (&dk)[4], f32x16 (&dv)[4]) {
  constexpr unsigned slot = U * kTileBytes;
  constexpr unsigned sslot = U * kStatBytes;
  wait_vmcnt<kDkvOps * (kAhead - 1)>();
  barrier_lds();
  if (n_t > 1) kv_load(cx, t + kAhead, ln.lane);  // a single-tile segment needs no prefetch
  // S = Q K^T - LSE / scale and dP = dO V^T - D: lane = key l32, element v = query
  // 8 (v / 4) + 4 h32 + v % 4, whose stats are the 4 consecutive floats at 8 (v / 4) + 4 h32.
  // One sequence of 32 MFMAs: n = 0..7 S (Q rows), 8..15 dP (dO rows) with P's exp2 work,
  // 16..23 dV^T += dO^T P with dS's work, 24..31 dK^T += Q^T dS. Every LDS operand is read
  // two MFMAs ahead of its use; scheduling barriers hold the order.
  bf16x8 op[32];
  // The row-read base is made opaque per step and again before the dO rows, so the compiler
  // forms each step's address where it is read rather than keeping eight of them live.
  unsigned r0 = ln.raddr0;
  asm volatile("" : "+v"(r0));
  auto read = [&](int n) {
    if (n < 8) op[n] = lds_row((r0 ^ (n << 5)) + slot);
    else if (n < 16) op[n] = lds_row((r0 ^ ((n - 8) << 5)) + slot + kRing);
    else if (n < 24) op[n] = tr_operand(ln.qtaddr, slot + kRing, n - 16);
    else op[n] = tr_operand(ln.qtaddr, slot, n - 24);
  };
  f32x16 S, dP;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const f32x4 ls = *(lds_f32x4*)(uintptr_t)(ln.staddr + sslot + 32 * a);
#pragma unroll
    for (int b = 0; b < 4; ++b) S[4 * a + b] = ls[b];
  }
  read(0);
  read(1);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const f32x4 nd = *(lds_f32x4*)(uintptr_t)(ln.staddr + sslot + 32 * a + kBT * 4);
#pragma unroll
    for (int b = 0; b < 4; ++b) dP[4 * a + b] = nd[b];
  }
  sched_fence();
  // P and dS are formed in place of S and dP (fewer live registers).
  u32x4 pb[2], sb[2];
  bf16x8 P[2], dS[2];
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    if (n == 6) asm volatile("" : "+v"(r0));
    if (n + 2 < 32) read(n + 2);
    sched_fence();
    if (n < 8) {
      S = mfma(op[n], kr[n], S);
      if (n == 7 && t == n_t - 1) {
        sched_fence();
        mask_last_tile(S, cx.seg_len, n_t, ln.h32);
      }
    } else if (n < 16) {
      const int s = n - 8;
      dP = mfma(op[n], vr[s], dP);
      sched_fence();
      S[2 * s] = __builtin_amdgcn_exp2f(S[2 * s] * c);
      S[2 * s + 1] = __builtin_amdgcn_exp2f(S[2 * s + 1] * c);
      pack_pair(pb, s, S[2 * s], S[2 * s + 1]);
      if (s == 3) P[0] = __builtin_bit_cast(bf16x8, pb[0]);
      if (s == 7) P[1] = __builtin_bit_cast(bf16x8, pb[1]);
    } else if (n < 24) {
      const int i = n - 16;
      dv[i & 3] = mfma(op[n], P[i >> 2], dv[i & 3]);
      sched_fence();
      pack_pair(sb, i, S[2 * i] * dP[2 * i], S[2 * i + 1] * dP[2 * i + 1]);
      if (i == 3) dS[0] = __builtin_bit_cast(bf16x8, sb[0]);
      if (i == 7) dS[1] = __builtin_bit_cast(bf16x8, sb[1]);
    } else {
      const int i = n - 24;
      dk[i & 3] = mfma(op[n], dS[i >> 2], dk[i & 3]);
    }
    sched_fence();
  }
}

__device__ __forceinline__ void store_rows_t(uint16_t* orow, const f32x16 (&acc)[4], float mul, int h32) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 tmp[2];
      pack_pair(tmp, 0, acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
      pack_pair(tmp, 1, acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
      u32x2 pk;
      pk[0] = tmp[0][0];
      pk[1] = tmp[0][1];
      *(u32x2*)(orow + 32 * db + 8 * g + 4 * h32) = pk;
    }
}

// dK and dV for the 256 keys of work item w.
__device__ __forceinline__ void dkdv_body(const Work& w, const uint16_t* __restrict__ q,
                                          const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                          const uint16_t* __restrict__ dout, const float* __restrict__ ws_nl,
                                          const float* __restrict__ ws_d, uint16_t* __restrict__ dk,
                                          uint16_t* __restrict__ dv, int n_heads, int64_t total_tokens, float c,
                                          float scale) {
  extern __shared__ __attribute__((aligned(1024))) char smem_generic[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned lds_base = (unsigned)(uintptr_t)(lds_char*)smem_generic;

  KvCtx cx;
  cx.row_stride = (unsigned)n_heads * kRowBytes;
  cx.qbase = (const char*)q + ((int64_t)w.seg_start * n_heads + w.head) * kRowBytes;
  cx.dobase = (const char*)dout + ((int64_t)w.seg_start * n_heads + w.head) * kRowBytes;
  cx.nlbase = (const char*)(ws_nl + (int64_t)w.head * total_tokens + w.seg_start);
  cx.dbase = (const char*)(ws_d + (int64_t)w.head * total_tokens + w.seg_start);
  cx.seg_len = w.seg_len;
  cx.lds_copy = lds_base + wave * 1024;
  // Stats: waves 0..3 copy -LSE / scale, waves 4..7 copy -D; wave w's 8 lanes copy floats
  // 8 (w % 4) .. +7 of the tile.
  cx.statbase = (wave < 4 ? cx.nlbase : cx.dbase) + 32 * (wave & 3);  // floats 8 (w % 4) ..
  cx.lds_stat = lds_base + 4 * kRing + (wave < 4 ? 0 : kBT * 4) + 32 * (wave & 3);
  cx.stat_row = 8 * (wave & 3) + (lane & 7);
  row_copy_lane(wave, lane, cx.rrow, cx.roff);
  tr_copy_lane(wave, lane, cx.trow, cx.toff);
  cx.rconst = (unsigned)cx.rrow * cx.row_stride + cx.roff;
  cx.tconst = (unsigned)cx.trow * cx.row_stride + cx.toff;

  KvLane ln;
  ln.lane = lane;
  ln.h32 = lane >> 5;
  ln.l32 = lane & 31;
  ln.raddr0 = row_read_addr(lds_base, ln.l32, ln.h32, 0);
  ln.qtaddr = tr_read_base(lds_base + 2 * kRing, lane);
  ln.staddr = lds_base + 4 * kRing + 4 * (4 * ln.h32);

  // This lane's key: K and V as B operands (k[key][16 s + 8 h32 .. +7]).
  int key = w.r0 + wave * 32 + ln.l32;
  const bool live = key < w.seg_len;
  key = live ? key : w.seg_len - 1;
  const int64_t tok = (int64_t)w.seg_start + key;
  bf16x8 kr[8], vr[8];
  {
    const int64_t off = (tok * n_heads + w.head) * kD + ln.h32 * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kr[s] = *(const bf16x8*)(k + off + 16 * s);
      vr[s] = *(const bf16x8*)(v + off + 16 * s);
    }
  }
  // Wait for K and V here, before any tile copy is issued. Left to the compiler, that wait
  // sat at their first use inside the tile loop, where it also counted the copies of the
  // tiles ahead and so drained the prefetch on every tile.
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(kr[s]), "v"(vr[s]));
  f32x16 dka[4], dva[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }
  const int n_t = (w.seg_len + kBT - 1) / kBT;
  if (w.seg_len >= kBT) {
#pragma unroll
    for (int t = 0; t < kAhead; ++t) kv_load(cx, t, lane);
  } else {
    kv_load_short(cx, lane, wave);
    // As in the dQ kernel: the steps' waits leave more copies in flight than one tile issues.
    wait_vmcnt<0>();
  }
  for (int t = 0; t < n_t; t += kSlots) {
    kv_step<0>(cx, ln, t, n_t, kr, vr, c, dka, dva);
    if (t + 1 < n_t) kv_step<1>(cx, ln, t + 1, n_t, kr, vr, c, dka, dva);
    if (t + 2 < n_t) kv_step<2>(cx, ln, t + 2, n_t, kr, vr, c, dka, dva);
    if (t + 3 < n_t) kv_step<3>(cx, ln, t + 3, n_t, kr, vr, c, dka, dva);
  }
  wait_vmcnt<0>();

  if (live) {
    store_rows_t(dk + (tok * n_heads + w.head) * kD, dka, scale, ln.h32);
    store_rows_t(dv + (tok * n_heads + w.head) * kD, dva, 1.0f, ln.h32);
  }
}

// Both gradient passes in one launch: blocks [0, 8 P) are the dK/dV pass and blocks [8 P, 16 P)
// the dQ pass (P = ceil(n_logical / 8) blocks per XCD in each; the second pass starts at a
// multiple of 8, so its blocks keep their XCDs, and XCD x's tiles of both passes are the same
// (head, segment) tiles). The passes are independent (both read only the inputs and the prep
// kernel's statistics), and the dQ blocks, dispatched after the dK/dV ones, fill the compute
// units that the dK/dV pass's last, partial round leaves idle. LDS: the larger of the two
// passes' (the dK/dV ring).
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                const uint16_t* __restrict__ dout, const float* __restrict__ ws_nl, const float* __restrict__ ws_d,
                uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                const int32_t* __restrict__ cu_seqlens, int n_seqs, int tiles_per_seq, int max_seqlen, int n_heads,
                int64_t total_tokens, float c, float scale, int n_logical) {
  const int per_xcd = (n_logical + 7) >> 3;
  const int b = blockIdx.x;
  if (b < 8 * per_xcd) {
    const Work w = map_block(b, per_xcd, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, total_tokens, n_logical);
    if (w.ok) dkdv_body(w, q, k, v, dout, ws_nl, ws_d, dk, dv, n_heads, total_tokens, c, scale);
  } else {
    const Work w =
        map_block(b - 8 * per_xcd, per_xcd, cu_seqlens, n_seqs, tiles_per_seq, max_seqlen, total_tokens, n_logical);
    if (w.ok) dq_body(w, q, k, v, dout, ws_nl, ws_d, dq, n_heads, total_tokens, c, scale);
  }
}

// File-scope scratch for lsv_attn_bwd_noalloc: the prep kernel's two fp32 values per (head,
// token) for callers that cannot allocate. 2^27 bytes hold 2^24 (token, head) rows, e.g. one
// 299,593-token segment at 56 heads, the largest the 32-bit offsets allow. Each GPU the library
// runs on holds its own copy until the process ends. In host code the name stands for a host-side
// shadow, not a device address: kernels get the per-device address from scratch_address().
constexpr int64_t kScratchBytes = (int64_t)1 << 27;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that `stream` belongs to (the current device
// for the null stream), looked up once per device with that device current.
int scratch_address(hipStream_t stream, float** out) {
  int dev = 0;
  if (stream == nullptr) {
    if (hipGetDevice(&dev) != hipSuccess) return LSV_ERR_HIP;
  } else if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    return LSV_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return LSV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return LSV_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return LSV_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return LSV_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return LSV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = (float*)g_scratch_ptr[dev];
  return LSV_OK;
}

constexpr int kProceed = 1;  // bwd_checks: arguments valid and there is work to launch

// The backward's argument checks, before any HIP call (the workspace aside): a status to
// return, or kProceed.
int bwd_checks(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
               int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale) {
  if (n_seqs < 0 || max_seqlen < 0 || total_tokens < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (n_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return LSV_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return LSV_ERR_ALIGNMENT;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens) & 3) return LSV_ERR_ALIGNMENT;
  if (total_tokens > (int64_t)INT32_MAX || total_tokens * (int64_t)n_heads >= ((int64_t)1 << 31))
    return LSV_ERR_UNSUPPORTED;
  const int64_t row_stride = (int64_t)n_heads * kRowBytes;
  if (row_stride >= (1 << 24) || (int64_t)max_seqlen >= (1 << 24) ||
      (int64_t)max_seqlen * row_stride + kRowBytes > (int64_t)UINT32_MAX)
    return LSV_ERR_UNSUPPORTED;
  const int64_t tiles = ((int64_t)max_seqlen + kBlockRows - 1) / kBlockRows;
  if (2 * ((tiles * n_seqs * (int64_t)n_heads + 7) / 8 * 8) > (int64_t)INT32_MAX) return LSV_ERR_UNSUPPORTED;
  return kProceed;
}

// The two kernels on `stream`, with the stats in ws (2 * total_tokens * n_heads floats, fully
// overwritten by the prep kernel before the other two read them). Arguments already checked.
int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
               int64_t total_tokens, int32_t n_heads, float scale, float* ws, hipStream_t st) {
  const int64_t tiles = ((int64_t)max_seqlen + kBlockRows - 1) / kBlockRows;
  const int64_t n_logical = tiles * n_seqs * (int64_t)n_heads;
  const int64_t grid = (n_logical + 7) / 8 * 8;
  static_assert(kDkvLds >= kDqLds, "the merged launch sizes LDS for the dK/dV pass");
  if (hipFuncSetAttribute((const void*)attn_bwd_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kDkvLds) !=
      hipSuccess)
    return LSV_ERR_HIP;
  float* ws_nl = ws;
  float* ws_d = ws_nl + total_tokens * (int64_t)n_heads;
  const float c = (float)((double)scale * 1.4426950408889634074);
  const int64_t rows = total_tokens * (int64_t)n_heads;
  const int64_t prep_need = (rows + 15) / 16;
  const int64_t prep_grid = prep_need < (1 << 22) ? prep_need : (1 << 22);
  (void)hipGetLastError();
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)prep_grid), dim3(256), 0, st, (const u32x4*)o,
                     (const u32x4*)dout, lse, ws_nl, ws_d, (unsigned)rows, (unsigned)n_heads, total_tokens,
                     (float)(1.0 / (double)scale));
  hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)(2 * grid)), dim3(kThreads), kDkvLds, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, ws_nl, ws_d, (uint16_t*)dq,
                     (uint16_t*)dk, (uint16_t*)dv, cu_seqlens, (int)n_seqs, (int)tiles, (int)max_seqlen,
                     (int)n_heads, total_tokens, c, scale, (int)n_logical);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

}  // namespace

extern "C" {

int64_t lsv_attn_bwd_workspace_size(int64_t total_tokens, int32_t n_heads) {
  if (total_tokens < 0 || n_heads < 1) return -1;
  return 2 * total_tokens * (int64_t)n_heads * (int64_t)sizeof(float);
}

int lsv_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                 int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale, void* workspace,
                 int64_t workspace_bytes, void* stream) {
  const int rc = bwd_checks(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen, total_tokens,
                            n_heads, head_dim, scale);
  if (rc != kProceed) return rc;
  if (!workspace) return LSV_ERR_INVALID_ARG;
  if ((uintptr_t)workspace & 3) return LSV_ERR_ALIGNMENT;
  if (workspace_bytes < lsv_attn_bwd_workspace_size(total_tokens, n_heads)) return LSV_ERR_INVALID_ARG;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, scale,
                    (float*)workspace, (hipStream_t)stream);
}

int64_t lsv_attn_bwd_noalloc_max_rows(void) { return kScratchBytes / (2 * (int64_t)sizeof(float)); }

int lsv_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs,
                         int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale,
                         void* stream) {
  const int rc = bwd_checks(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen, total_tokens,
                            n_heads, head_dim, scale);
  if (rc != kProceed) return rc;
  if (lsv_attn_bwd_workspace_size(total_tokens, n_heads) > kScratchBytes) return LSV_ERR_UNSUPPORTED;
  float* ws = nullptr;
  const int src = scratch_address((hipStream_t)stream, &ws);
  if (src != LSV_OK) return src;
  return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, scale,
                    ws, (hipStream_t)stream);
}

}  // extern "C"
