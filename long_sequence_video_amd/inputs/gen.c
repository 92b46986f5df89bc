/* Seeded synthetic inputs for the attention forward: bf16 bit patterns.
 *
 * This generator serves both the HIP path and the fp64 oracle; it holds none
 * of the attention arithmetic. Every value is a pure function of
 * (seed, tensor id, element index), so the output does not depend on the
 * number of threads.
 *
 * Definitions:
 *   splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014): state advances by the golden gamma
 *   0x9E3779B97F4A7C15 and each output is the state passed through the
 *   variant-13 mix. Output i (i >= 0) of a stream whose state starts at s0 is
 *   mix(s0 + (i + 1) * gamma).
 *   Stream start for (seed, tensor): s0 = output number `tensor` of the stream
 *   whose state starts at `seed`.
 *   Standard normals by the Box-Muller transform (Box and Muller, 1958): pair p
 *   takes outputs a = 2p and b = 2p + 1, u1 = ((a >> 11) + 1) * 2^-53 in (0, 1],
 *   u2 = (b >> 11) * 2^-53 in [0, 1), r = sqrt(-2 ln u1), t = 2 pi u2; element
 *   2p is r cos t and element 2p + 1 is r sin t, computed in double.
 *   Each double is rounded to float (nearest even), then to bf16 (nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "lsvgen.h"

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_at(uint64_t s0, uint64_t i) { return mix64(s0 + (i + 1) * GAMMA); }

static inline uint64_t stream_start(uint64_t seed, uint32_t tensor) { return stream_at(seed, tensor); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Two standard normals for pair p of stream s0. */
static inline void normal_pair(uint64_t s0, uint64_t p, double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t a = stream_at(s0, 2 * p), b = stream_at(s0, 2 * p + 1);
  double u1 = (double)((a >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(b >> 11) * 0x1.0p-53;
  double r = sqrt(-2.0 * log(u1)), t = two_pi * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

/* out[e] = bf16(N(0,1)) for e in [0, n). Returns 0, or -1 on bad arguments. */
int lsvgen_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint32_t tensor) {
  if (n < 0 || (n > 0 && !out)) return -1;
  const uint64_t s0 = stream_start(seed, tensor);
  const int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < pairs; ++p) {
    double z0, z1;
    normal_pair(s0, (uint64_t)p, &z0, &z1);
    out[2 * p] = f32_to_bf16_rne((float)z0);
    if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16_rne((float)z1);
  }
  return 0;
}

/* In place, per row of `row_len` bf16 values: x <- bf16(x * (mean(x^2) + eps)^-1/2),
 * the scale computed in double from the bf16 values (unit weight). */
int lsvgen_rms_normalize_bf16(uint16_t* x, int64_t rows, int32_t row_len, double eps) {
  if (rows < 0 || row_len <= 0 || (rows > 0 && !x)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint16_t* row = x + r * (int64_t)row_len;
    double ss = 0.0;
    for (int32_t i = 0; i < row_len; ++i) {
      double v = bf16_to_f32(row[i]);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / row_len + eps);
    for (int32_t i = 0; i < row_len; ++i) row[i] = f32_to_bf16_rne((float)((double)bf16_to_f32(row[i]) * inv));
  }
  return 0;
}

/* `n_choose` distinct indices from [0, n_total), by a partial Fisher-Yates shuffle
 * driven by the (seed, tensor) stream: step i swaps slot i with slot
 * i + floor(w_i * (n_total - i) / 2^64), w_i = output i. Sorted ascending on return.
 * `work` must hold n_total int64 values. */
int lsvgen_choose(int64_t* out, int64_t n_choose, int64_t n_total, int64_t* work, uint64_t seed, uint32_t tensor) {
  if (n_choose < 0 || n_total < 0 || n_choose > n_total || (n_total > 0 && !work) || (n_choose > 0 && !out))
    return -1;
  const uint64_t s0 = stream_start(seed, tensor);
  for (int64_t i = 0; i < n_total; ++i) work[i] = i;
  for (int64_t i = 0; i < n_choose; ++i) {
    uint64_t w = stream_at(s0, (uint64_t)i);
    int64_t j = i + (int64_t)(((__uint128_t)w * (uint64_t)(n_total - i)) >> 64);
    int64_t t = work[i];
    work[i] = work[j];
    work[j] = t;
  }
  /* insertion sort of the chosen prefix (n_choose is small) */
  for (int64_t i = 0; i < n_choose; ++i) out[i] = work[i];
  for (int64_t i = 1; i < n_choose; ++i) {
    int64_t v = out[i], j = i - 1;
    while (j >= 0 && out[j] > v) { out[j + 1] = out[j]; --j; }
    out[j + 1] = v;
  }
  return 0;
}

/* Multiply rows[i] (each `row_len` bf16 values) by `factor`, rounding to bf16.
 * A power-of-two factor is exact unless it overflows. */
int lsvgen_scale_rows_bf16(uint16_t* x, const int64_t* rows, int64_t n_rows, int64_t row_len, float factor) {
  if (n_rows < 0 || row_len < 0 || (n_rows > 0 && (!x || !rows))) return -1;
  for (int64_t i = 0; i < n_rows; ++i) {
    uint16_t* row = x + rows[i] * row_len;
    for (int64_t j = 0; j < row_len; ++j) row[j] = f32_to_bf16_rne(bf16_to_f32(row[j]) * factor);
  }
  return 0;
}

/* Element e of the (seed, tensor) normal stream as a double (before rounding). */
double lsvgen_normal_f64_at(uint64_t seed, uint32_t tensor, int64_t e) {
  double z0, z1;
  normal_pair(stream_start(seed, tensor), (uint64_t)(e / 2), &z0, &z1);
  return (e & 1) ? z1 : z0;
}

/* Per-tensor e4m3 quantisation of bf16 values: out[i] = e4m3(x[i] / descale), OCP FP8 E4M3
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities), rounded to nearest
 * with ties to even in the binade of |y| (subnormal spacing 2^-9 below 2^-6), saturating at
 * 448; the division is done in double. Exactly what inputs.f64_to_e4m3_bits gives for
 * x / descale, without its float64 temporaries. */
int lsvgen_quantize_e4m3_bf16(const uint16_t* x, int64_t n, double descale, uint8_t* out) {
  if (n < 0 || (n > 0 && (!x || !out)) || !(descale > 0.0) || !isfinite(descale)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double y = (double)bf16_to_f32(x[i]) / descale;
    const uint8_t sign = signbit(y) ? 0x80 : 0;
    double a = fabs(y);
    if (a > 448.0) a = 448.0;
    uint8_t bits = 0;
    if (a > 0.0) {
      int ex;
      frexp(a, &ex);             /* a = f 2^ex, f in [0.5, 1): the binade is 2^(ex - 1) */
      int e = ex - 1;
      if (e < -6) e = -6;        /* subnormals share the spacing of the lowest binade */
      if (e > 8) e = 8;
      const double quantum = ldexp(1.0, e - 3);
      double r = rint(a / quantum) * quantum;   /* default rounding: to nearest, ties to even */
      if (r > 448.0) r = 448.0;
      if (r >= 0.015625) {       /* normal: r = (1 + m/8) 2^ee */
        int er;
        frexp(r, &er);
        const int ee = er - 1;
        const int mant = (int)(ldexp(r, -ee) * 8.0 - 8.0);
        bits = (uint8_t)(((ee + 7) << 3) | mant);
      } else {                   /* subnormal: r = m 2^-9 */
        bits = (uint8_t)(int)ldexp(r, 9);
      }
    }
    out[i] = (uint8_t)(bits | sign);
  }
  return 0;
}

/* The largest |x| over n bf16 values, as a double (0 for n = 0). */
int lsvgen_amax_bf16(const uint16_t* x, int64_t n, double* amax) {
  if (n < 0 || (n > 0 && !x) || !amax) return -1;
  uint16_t m = 0;
#pragma omp parallel for reduction(max : m) schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t u = (uint16_t)(x[i] & 0x7FFF);   /* magnitudes order like their bit patterns */
    if (u > m) m = u;
  }
  *amax = (double)bf16_to_f32(m);
  return 0;
}
