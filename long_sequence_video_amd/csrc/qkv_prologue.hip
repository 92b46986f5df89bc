// Fused QKV prologue for gfx950 (MI355X): per-head RMSNorm + partial rotate-half RoPE of Q
// and K, and a copy of V, written as one stacked [3, B, S, H, D] buffer.
//
// The operation is the MotionKernel qkv_prologue of FastVideo #2049 (diff of
// fastvideo/models/dits/minimax_h3_fusions/mk/qkv_prologue.py, module docstring and kernel):
// every (token, head) row x of Q (and of K, with its own weight) becomes
//   y_i = x_i * rsqrt(mean(x^2) + eps) * w_i
//   out_i = y_i cos_i - y_{i+R/2} sin_i   (i < R/2)
//   out_i = y_i cos_i + y_{i-R/2} sin_i   (R/2 <= i < R)
//   out_i = y_i                           (i >= R)
// with the cos/sin row of the token's position in its sequence; fp32 arithmetic, one
// rounding to bf16 at the store. V is copied bit for bit.
//
// Design: the pass streams every byte once (read q, k, v; write three planes), so it is
// bound by HBM. A row of 128 channels (256 bytes) belongs to 16 consecutive lanes, 8
// channels (one 16-byte load) each; a wave holds 4 rows, a 256-thread block 16. The RMS
// sum is reduced over the 16 lanes with xor shuffles. The rotate-half partner of channel
// 8j+e is channel 8j+e +- R/2, i.e. the same e in lane j +- R/16 of the row, so one lane
// permute of the raw bf16 inputs (4 dwords) brings it in; the partner's weight is loaded
// once per thread. Each thread issues its three 16-byte loads (q, k, v) before it computes
// or stores anything. One block per 16 rows (a grid-stride loop only past 2^22 blocks, which
// keeps the launch under 2^32 work-items); stores are non-temporal, since nothing reads the
// output back soon enough to gain from the cache (measured: 6.1 vs 5.5 TB/s). Plane
// offsets are 64-bit (a plane of the 4 x 40,000 x 56 x 128 batch exceeds 2^30 elements,
// the second plane starts past 2^31).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "lsv.h"

namespace {

constexpr int kD = 128;
constexpr int kLanesPerRow = 16;                    // 8 bf16 channels per lane
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;  // 16
constexpr int64_t kMaxGrid = 1 << 22;              // blocks per launch (x 256 < 2^32 work-items)

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ float lo_f(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const u32x4& u, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = lo_f(u[i]);
    f[2 * i + 1] = hi_f(u[i]);
  }
}

__device__ __forceinline__ unsigned pack2(float a, float b) {
  bf16x2 p;
  p[0] = (__bf16)a;  // round to nearest even
  p[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, p);
}

// Sum over the 16 lanes of this row (lanes are grouped by 16 from lane 0 of the wave).
__device__ __forceinline__ float row_sum16(float x) {
  x += __shfl_xor(x, 8, kLanesPerRow);
  x += __shfl_xor(x, 4, kLanesPerRow);
  x += __shfl_xor(x, 2, kLanesPerRow);
  x += __shfl_xor(x, 1, kLanesPerRow);
  return x;
}

struct LaneConst {
  float wq[8], wk[8];    // this lane's weights
  float wqp[8], wkp[8];  // the partner lane's weights
  int partner;           // source lane (within the wave) of the rotate-half partner
  float sgn;             // -1 (first half), +1 (second half)
  bool rotates;          // this lane's channels are below R
};

// One row: normalise, rotate, round; returns the packed bf16 output (4 dwords).
__device__ __forceinline__ u32x4 norm_rope(const u32x4& xr, const float (&w)[8], const float (&wp)[8],
                                           const LaneConst& lc, const u32x4& cr, const u32x4& sr, float eps) {
  float x[8];
  unpack8(xr, x);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
  ss = row_sum16(ss);
  const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / kD) + eps);
  // partner's raw inputs (every lane takes part in the permute, rotating or not)
  u32x4 pr;
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = (unsigned)__shfl((int)xr[i], lc.partner, 64);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * w[e];
  u32x4 out;
  if (lc.rotates) {
    float xp[8], c[8], s[8];
    unpack8(pr, xp);
    unpack8(cr, c);
    unpack8(sr, s);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float yp = xp[e] * inv * wp[e];
      o[e] = __builtin_fmaf(yp, lc.sgn * s[e], y[e] * c[e]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack2(o[2 * i], o[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack2(y[2 * i], y[2 * i + 1]);
  }
  return out;
}

__global__ void __launch_bounds__(kThreads)
qkv_prologue_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                    const uint16_t* __restrict__ qw, const uint16_t* __restrict__ kw,
                    const u32x4* __restrict__ cosb, const u32x4* __restrict__ sinb, u32x4* __restrict__ out,
                    unsigned n_rows, unsigned n_heads, unsigned seq_len, int rotary_dim, int64_t plane_vec, float eps) {
  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);  // lane within the row: channels 8j .. 8j+7
  const int h16 = rotary_dim / 16;          // lanes per rotary half
  LaneConst lc;
  lc.rotates = j < 2 * h16;
  lc.sgn = j < h16 ? -1.0f : 1.0f;
  const int jp = !lc.rotates ? j : (j < h16 ? j + h16 : j - h16);
  lc.partner = (lane & ~(kLanesPerRow - 1)) | jp;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lc.wq[e] = __uint_as_float((unsigned)qw[8 * j + e] << 16);
    lc.wk[e] = __uint_as_float((unsigned)kw[8 * j + e] << 16);
    lc.wqp[e] = __uint_as_float((unsigned)qw[8 * jp + e] << 16);
    lc.wkp[e] = __uint_as_float((unsigned)kw[8 * jp + e] << 16);
  }
  const int rvec = rotary_dim / 8;          // 16-byte vectors per table row
  const unsigned stride = gridDim.x * kRowsPerBlock;
  const unsigned first = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);

  // The 16 lanes of a row share its loop bounds, so the row's shuffles never see an
  // inactive lane of the row.
  for (unsigned row = first; row < n_rows; row += stride) {
    const int64_t idx = (int64_t)row * (kD / 8) + j;
    const u32x4 xq = q[idx];
    const u32x4 xk = k[idx];
    const u32x4 xv = v[idx];
    u32x4 cr = {}, sr = {};
    if (lc.rotates) {
      const unsigned pos = (row / n_heads) % seq_len;
      cr = cosb[(int64_t)pos * rvec + j];
      sr = sinb[(int64_t)pos * rvec + j];
    }
    // V goes out first; Q, then K, each stored as soon as it is done (a scheduling barrier
    // keeps the two rows from being interleaved; measured 1.3% faster than storing all three
    // at the end).
    __builtin_nontemporal_store(xv, out + 2 * plane_vec + idx);
    const u32x4 oq = norm_rope(xq, lc.wq, lc.wqp, lc, cr, sr, eps);
    __builtin_nontemporal_store(oq, out + idx);
    __builtin_amdgcn_sched_barrier(0);
    const u32x4 ok = norm_rope(xk, lc.wk, lc.wkp, lc, cr, sr, eps);
    __builtin_nontemporal_store(ok, out + plane_vec + idx);
  }
}

// The same per-row step on one tensor: x [rows, 128] -> out, with one cos/sin table row per
// token (row / n_heads) -- the K side of a forward whose Q side is normalised in the attention
// kernel's Q load (lsv_attn_fwd_qnorm).
__global__ void __launch_bounds__(kThreads)
norm_rope_kernel(const u32x4* __restrict__ x, const uint16_t* __restrict__ w, const u32x4* __restrict__ cosb,
                 const u32x4* __restrict__ sinb, u32x4* __restrict__ out, unsigned n_rows, unsigned n_heads,
                 int rotary_dim, float eps) {
  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);
  const int h16 = rotary_dim / 16;
  LaneConst lc;
  lc.rotates = j < 2 * h16;
  lc.sgn = j < h16 ? -1.0f : 1.0f;
  const int jp = !lc.rotates ? j : (j < h16 ? j + h16 : j - h16);
  lc.partner = (lane & ~(kLanesPerRow - 1)) | jp;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lc.wq[e] = __uint_as_float((unsigned)w[8 * j + e] << 16);
    lc.wqp[e] = __uint_as_float((unsigned)w[8 * jp + e] << 16);
  }
  const int rvec = rotary_dim / 8;
  const unsigned stride = gridDim.x * kRowsPerBlock;
  const unsigned first = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  for (unsigned row = first; row < n_rows; row += stride) {
    const int64_t idx = (int64_t)row * (kD / 8) + j;
    const u32x4 xr = x[idx];
    u32x4 cr = {}, sr = {};
    if (lc.rotates) {
      const unsigned tok = row / n_heads;
      cr = cosb[(int64_t)tok * rvec + j];
      sr = sinb[(int64_t)tok * rvec + j];
    }
    __builtin_nontemporal_store(norm_rope(xr, lc.wq, lc.wqp, lc, cr, sr, eps), out + idx);
  }
}

}  // namespace

extern "C" int lsv_norm_rope(const void* x, const void* weight, const void* cos, const void* sin, void* out,
                             int64_t total_tokens, int32_t n_heads, int32_t head_dim, int32_t rotary_dim, float eps,
                             void* stream) {
  if (total_tokens < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (rotary_dim < 0 || rotary_dim > kD || rotary_dim % 16 != 0) return LSV_ERR_UNSUPPORTED;
  if (total_tokens == 0) return LSV_OK;
  if (!x || !weight || !out) return LSV_ERR_INVALID_ARG;
  if (rotary_dim > 0 && (!cos || !sin)) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)x | (uintptr_t)out | (uintptr_t)cos | (uintptr_t)sin) & 15) return LSV_ERR_ALIGNMENT;
  if ((uintptr_t)weight & 1) return LSV_ERR_ALIGNMENT;
  const int64_t rows = total_tokens * (int64_t)n_heads;
  if (total_tokens >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31)) return LSV_ERR_UNSUPPORTED;
  const int64_t need = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t grid = need < kMaxGrid ? need : kMaxGrid;
  (void)hipGetLastError();
  hipLaunchKernelGGL(norm_rope_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream, (const u32x4*)x,
                     (const uint16_t*)weight, (const u32x4*)cos, (const u32x4*)sin, (u32x4*)out, (unsigned)rows,
                     (unsigned)n_heads, (int)rotary_dim, eps);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}

extern "C" int lsv_qkv_prologue(const void* q, const void* k, const void* v, const void* q_weight,
                                const void* k_weight, const void* cos, const void* sin, void* out, int64_t batch,
                                int64_t seq_len, int32_t n_heads, int32_t head_dim, int32_t rotary_dim, float eps,
                                void* stream) {
  if (batch < 0 || seq_len < 0 || n_heads < 1) return LSV_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return LSV_ERR_INVALID_ARG;
  if (head_dim != kD) return LSV_ERR_UNSUPPORTED;
  if (rotary_dim < 0 || rotary_dim > kD || rotary_dim % 16 != 0) return LSV_ERR_UNSUPPORTED;
  if (batch == 0 || seq_len == 0) return LSV_OK;
  if (!q || !k || !v || !q_weight || !k_weight || !out) return LSV_ERR_INVALID_ARG;
  if (rotary_dim > 0 && (!cos || !sin)) return LSV_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)cos | (uintptr_t)sin) & 15)
    return LSV_ERR_ALIGNMENT;
  if (((uintptr_t)q_weight | (uintptr_t)k_weight) & 1) return LSV_ERR_ALIGNMENT;
  if (batch >= ((int64_t)1 << 31) || seq_len >= ((int64_t)1 << 31)) return LSV_ERR_UNSUPPORTED;
  const int64_t tokens = batch * seq_len;  // < 2^62
  if (tokens >= ((int64_t)1 << 31)) return LSV_ERR_UNSUPPORTED;
  const int64_t rows = tokens * (int64_t)n_heads;  // < 2^62
  if (rows >= ((int64_t)1 << 31)) return LSV_ERR_UNSUPPORTED;
  const int64_t plane_vec = rows * (kD / 8);  // 16-byte vectors per plane
  const int64_t need = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t grid = need < kMaxGrid ? need : kMaxGrid;
  (void)hipGetLastError();
  hipLaunchKernelGGL(qkv_prologue_kernel, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)q, (const u32x4*)k, (const u32x4*)v, (const uint16_t*)q_weight,
                     (const uint16_t*)k_weight, (const u32x4*)cos, (const u32x4*)sin, (u32x4*)out, (unsigned)rows,
                     (unsigned)n_heads, (unsigned)seq_len, (int)rotary_dim, plane_vec, eps);
  if (hipGetLastError() != hipSuccess) return LSV_ERR_LAUNCH;
  return LSV_OK;
}
