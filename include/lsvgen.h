/* lsvgen: the seeded synthetic-input generator (host C ABI, liblsvgen.so).
 *
 * The pages measure attention on MiniMax-H3 video clips (TensorRT-LLM PR #21275,
 * Description: 19k-104k packed tokens, 56 heads x 128; FastVideo compare
 * perf/ulysses-h3-adaptive: the sp=4 rank's 14-head share). No clip, prompt or
 * checkpoint is available, so inputs of those shapes are drawn from this generator.
 * It serves both the attention library and the fp64 test oracle and holds none of
 * the attention arithmetic.
 *
 * Every value is a pure function of (seed, tensor id, element index), so results do
 * not depend on the number of threads:
 *   - splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014). Output i of the stream whose state starts at s0 is
 *     mix(s0 + (i + 1) * 0x9E3779B97F4A7C15). The stream of (seed, tensor) starts at
 *     output number `tensor` of the stream whose state starts at `seed`.
 *   - Box-Muller (1958). Pair p takes outputs 2p and 2p + 1:
 *     u1 = ((a >> 11) + 1) 2^-53, u2 = (b >> 11) 2^-53, r = sqrt(-2 ln u1),
 *     t = 2 pi u2. Element 2p is r cos t and element 2p + 1 is r sin t, in double.
 *   - The double is rounded to float, then to bf16 (both to nearest even).
 *
 * Tensor ids: Q = 0, K = 1, V = 2, the boosted-row choice = 3; the prologue's norm
 * weights and its cos / sin tables use 4 .. 7.
 *
 * All pointers are host pointers owned by the caller. The functions allocate nothing
 * and are reentrant (loops run under OpenMP). Return value 0 means success and -1
 * means bad arguments (negative sizes, or a null pointer with a nonzero size); on -1
 * nothing is written.
 */
#ifndef LSVGEN_H
#define LSVGEN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* out[e] = bf16 bits of element e of the (seed, tensor) normal stream, e in [0, n). */
int lsvgen_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint32_t tensor);

/* In place, for each of `rows` rows of `row_len` bf16 values:
 * x <- bf16(x * (mean(x^2) + eps)^(-1/2)), with the scale computed in double from the
 * bf16 values (unit weight). This is the per-head RMS-normalised Q/K of the workloads. */
int lsvgen_rms_normalize_bf16(uint16_t* x, int64_t rows, int32_t row_len, double eps);

/* `n_choose` distinct indices of [0, n_total), sorted ascending, by a partial
 * Fisher-Yates shuffle: step i swaps slot i with slot i + floor(w_i (n_total - i) / 2^64),
 * where w_i is output i of the (seed, tensor) stream. `work` holds n_total int64 values
 * (scratch). Used for the boosted-key rows. */
int lsvgen_choose(int64_t* out, int64_t n_choose, int64_t n_total, int64_t* work, uint64_t seed, uint32_t tensor);

/* Multiplies rows rows[0 .. n_rows) of x (each row_len bf16 values) by `factor`,
 * rounding to bf16 (exact for a power of two unless it overflows). */
int lsvgen_scale_rows_bf16(uint16_t* x, const int64_t* rows, int64_t n_rows, int64_t row_len, float factor);

/* out[i] = OCP FP8 e4m3 bits of x[i] / descale (division in double; rounded to nearest, ties
 * to even, in the binade of the quotient, subnormal spacing 2^-9, saturating at +-448). The
 * per-tensor quantisation of the FP8 workloads (descale = fp32(amax / 448)). Returns -1 for
 * a negative n, null pointers or a descale that is not finite and positive. */
int lsvgen_quantize_e4m3_bf16(const uint16_t* x, int64_t n, double descale, uint8_t* out);

/* *amax = the largest |x[i]| of n bf16 values (0 for n = 0). */
int lsvgen_amax_bf16(const uint16_t* x, int64_t n, double* amax);

/* Element e of the (seed, tensor) normal stream as a double, before any rounding. */
double lsvgen_normal_f64_at(uint64_t seed, uint32_t tensor, int64_t e);

#ifdef __cplusplus
}
#endif

#endif /* LSVGEN_H */
