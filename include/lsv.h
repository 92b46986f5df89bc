/* lsv: dense non-causal varlen attention for AMD MI355X (gfx950): the BF16 forward and backward,
 * an FP8 (e4m3) forward, and the fused QKV prologue (QK RMSNorm + partial RoPE) that feeds them.
 *
 * The operation (FastVideo #2049, diff of fastvideo/attention/utils/flash_attn_cute.py,
 * the varlen forward wrapper; TensorRT-LLM PR #21275, Description): for every packed
 * segment [a, b) = [cu_seqlens[s], cu_seqlens[s+1]), every head h and every query row
 * i in [a, b),
 *     z_ij     = scale * sum_d q[i,h,d] k[j,h,d]      (keys j of the same segment only)
 *     O[i,h,:] = sum_j softmax_j(z_ij) v[j,h,:]
 *     LSE[h,i] = ln sum_j exp(z_ij)
 * Non-causal, no window, no softcap, one split (the forward is deterministic: the same
 * inputs give bit-identical outputs on every run). The varlen test on the FastVideo
 * #2049 page fixes the layouts: q/k/v/out are [total_tokens, heads, head_dim] and LSE
 * is fp32 [heads, total_tokens]; one cu_seqlens vector serves queries and keys.
 *
 * All functions are plain C, return a status (0 = success, negative = error), never
 * print, never throw, and never allocate device memory (lsv_attn_bwd_noalloc's scratch array
 * is a static device variable, set up by the HIP runtime when the code is loaded).
 */
#ifndef LSV_H
#define LSV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lsv_status {
  LSV_OK = 0,
  LSV_ERR_INVALID_ARG = -1, /* null pointer, negative size, non-finite or non-positive scale */
  LSV_ERR_UNSUPPORTED = -2, /* head_dim other than 128, or sizes beyond the launch limits */
  LSV_ERR_ALIGNMENT = -3,   /* q/k/v/o not 16-byte aligned, lse/cu_seqlens not 4-byte aligned */
  LSV_ERR_LAUNCH = -4,      /* the kernel launch failed (hipGetLastError after the launch) */
  LSV_ERR_HIP = -5          /* another HIP runtime call failed (e.g. no device) */
};

/* Attention forward on the caller's stream (asynchronous; nothing is synchronised).
 *
 * q, k, v      device pointers, bf16 bit patterns, row-major [total_tokens, n_heads, head_dim],
 *              16-byte aligned. Read only. Values are assumed finite.
 * o            device pointer, bf16, same layout as q. Written for every token row that lies
 *              inside a segment (rounded to nearest even from fp32); other rows untouched.
 * lse          device pointer, fp32 [n_heads, total_tokens], natural log of the sum of
 *              exp(scaled logits). Written for the same rows as o.
 * cu_seqlens   device pointer, int32 [n_seqs + 1]: cu[0] = 0, non-decreasing,
 *              cu[n_seqs] <= total_tokens, every cu[s+1] - cu[s] <= max_seqlen. It is never read
 *              on the host. A segment that breaks the bounds (cu[s] < 0, cu[s+1] < cu[s] or
 *              cu[s+1] > total_tokens) or is longer than max_seqlen is skipped: none of its
 *              rows is written and nothing outside [0, total_tokens) is read.
 * n_seqs       number of segments (>= 0). 0 is a successful no-op.
 * max_seqlen   upper bound of the segment lengths (>= 0); sizes the grid. 0 is a no-op.
 *              The kernel addresses one head's K/V rows of a segment with 32-bit byte
 *              offsets: max_seqlen * n_heads * head_dim * 2 must stay below 2^32 (e.g.
 *              max_seqlen <= 299,593 at 56 heads), else LSV_ERR_UNSUPPORTED.
 * total_tokens rows of q/k/v/o and columns of lse (>= 0).
 * n_heads      >= 1.
 * head_dim     must be 128.
 * scale        softmax scale applied to q.k in fp32 (finite, > 0); e.g. 1/sqrt(128).
 * stream       a hipStream_t, or NULL for the default stream.
 *
 * The caller owns every buffer; the library keeps no pointer after the call returns.
 * Validation happens before any HIP call; on error nothing is launched.
 */
int lsv_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                 int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                 float scale, void* stream);

/* Attention forward with the Q side of the QKV prologue fused into the Q-tile load
 * (asynchronous, one kernel on the caller's stream).
 *
 * The operation: the MotionKernel qkv_prologue of FastVideo #2049 (diff of
 * fastvideo/models/dits/minimax_h3_fusions/mk/qkv_prologue.py, module docstring and kernel;
 * MiniMaxH3Attention.forward on the same page rotates 96 of the 128 channels) applied to q, then
 * the varlen forward of lsv_attn_fwd. Each raw (token t, head) row x of q becomes
 *     y_i = x_i * rsqrt(mean_d x_d^2 + eps) * q_weight_i
 *     q'_i = y_i cos[t,i] - y_{i+R/2} sin[t,i]  (i < R/2),  y_i cos[t,i] + y_{i-R/2} sin[t,i]  (R/2 <= i < R),
 *     q'_i = y_i  (i >= R),
 * computed in fp32 and rounded once to bf16 -- the same steps and summation order as
 * lsv_norm_rope and lsv_qkv_prologue, so q' is bit-identical to what they write -- and
 * O, LSE = attention(q', k, v) exactly as lsv_attn_fwd computes it. Q is read once and never
 * written back: the prologue's pass over Q never touches HBM. k is expected already normalised
 * and rotated (lsv_norm_rope), v as is.
 *
 * q            device pointer, bf16 raw queries [total_tokens, n_heads, head_dim], 16-byte aligned.
 * k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale, stream:
 *              as for lsv_attn_fwd (same layouts, limits and skipped-segment rule).
 * q_weight     device pointer, bf16 [head_dim] norm weight, 16-byte aligned.
 * cos, sin     device pointers, bf16 [total_tokens, rotary_dim], one row per token (row t serves
 *              token t of every head), 16-byte aligned; may be NULL when rotary_dim is 0.
 * rotary_dim   R: a multiple of 16 in [0, 128] (96 for the H3 blocks), else LSV_ERR_UNSUPPORTED.
 * eps          finite, >= 0 (1e-5 for the H3 blocks).
 */
int lsv_attn_fwd_qnorm(const void* q, const void* k, const void* v, const void* q_weight, const void* cos,
                       const void* sin, int32_t rotary_dim, float eps, void* o, float* lse,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens,
                       int32_t n_heads, int32_t head_dim, float scale, void* stream);

/* lsv_attn_fwd_qnorm launched as lsv_attn_fwd_tail launches the forward (asynchronous; one kernel,
 * plus the combine pass when it cuts tiles): the same Q-side prologue in the Q-tile load, the
 * query tiles of the whole rounds run as in lsv_attn_fwd_qnorm, and each XCD's tiles of its last,
 * partial round are cut into the key ranges of lsv_attn_fwd_tail_plan and merged as there. The
 * result is bit-identical to lsv_norm_rope(q) followed by lsv_attn_fwd_tail on the same
 * compute_units. When nothing is cut this is lsv_attn_fwd_qnorm itself and the workspace is not
 * used.
 *
 * q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens, n_seqs, max_seqlen,
 * total_tokens, n_heads, head_dim, scale, stream: as for lsv_attn_fwd_qnorm.
 * compute_units, workspace, workspace_bytes: as for lsv_attn_fwd_tail.
 */
int lsv_attn_fwd_qnorm_tail(const void* q, const void* k, const void* v, const void* q_weight, const void* cos,
                            const void* sin, int32_t rotary_dim, float eps, void* o, float* lse,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens,
                            int32_t n_heads, int32_t head_dim, float scale, int32_t compute_units, void* workspace,
                            int64_t workspace_bytes, void* stream);

/* Workspace bytes lsv_attn_fwd_split needs for n_split key ranges: n_split partial rows of
 * head_dim + 1 fp32 values per (token, head), i.e. 4 * n_split * total_tokens * n_heads * 129;
 * 0 for n_split = 1. Returns -1 for a negative size, n_heads < 1 or n_split outside [1, 8]. */
int64_t lsv_attn_fwd_split_workspace_size(int64_t total_tokens, int32_t n_heads, int32_t n_split);

/* Attention forward with each segment's keys cut into n_split consecutive ranges
 * (asynchronous, two kernels on the caller's stream). The same operation as lsv_attn_fwd (the
 * varlen forward of FastVideo #2049), computed the way split-K attention combines partial
 * softmaxes: each (query tile, range) workgroup writes its range's normalised fp32 O_r and
 * LSE_r into the workspace, and a second pass writes, per row,
 *     LSE = ln sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r   (bf16, nearest even)
 * over the non-empty ranges. A range holds ceil(ceil(len / n_split) / 32) * 32 keys, the last
 * one the rest. More, shorter workgroups fill the last round of 256 compute units better when
 * a launch has few query tiles (e.g. 14 heads x 19,394 tokens: 1,064 workgroups); the result
 * differs from lsv_attn_fwd's by rounding only, and is deterministic.
 *
 * q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
 * stream: as for lsv_attn_fwd (same layouts, limits and skipped-segment rule).
 * n_split      1 to 8; 1 is lsv_attn_fwd itself (the workspace is not used).
 * workspace    device pointer, 16-byte aligned, at least lsv_attn_fwd_split_workspace_size
 *              bytes (else LSV_ERR_INVALID_ARG); overwritten. Owned by the caller.
 */
int lsv_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                       int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                       float scale, int32_t n_split, void* workspace, int64_t workspace_bytes, void* stream);

/* The key split that lsv_attn_fwd_tail applies for these sizes on compute_units workgroup slots
 * (one workgroup of 256 query rows per compute unit, compute_units / 8 on each of the 8 XCDs).
 * With n = ceil(max_seqlen / 256) * n_seqs * n_heads query tiles, each XCD owns P = ceil(n / 8)
 * consecutive tiles, as in lsv_attn_fwd (the last XCD fewer when n is not a multiple of 8); the
 * t = P mod (compute_units / 8) of them past its last whole round are cut into *n_split key
 * ranges when t is at most a quarter of a round -- as many ranges as fill the XCD's slots, at
 * most 8, each of at least 1024 keys of a max_seqlen-key segment -- and *n_tail_tiles = 8 t
 * (counting the last XCD's missing tiles, which cost nothing). Otherwise *n_split = 1 and
 * *n_tail_tiles = 0 (nothing is cut). compute_units must be a positive multiple of 8 (256 on
 * MI355X; lsv_device_peak reports it). Host-only arithmetic; LSV_ERR_INVALID_ARG on bad sizes. */
int lsv_attn_fwd_tail_plan(int32_t n_seqs, int32_t max_seqlen, int32_t n_heads, int32_t compute_units,
                           int32_t* n_split, int64_t* n_tail_tiles);

/* Workspace bytes lsv_attn_fwd_tail may need: compute_units * 256 rows * 129 fp32 values (an
 * upper bound for any sizes); -1 unless compute_units is a positive multiple of 8. */
int64_t lsv_attn_fwd_tail_workspace_size(int32_t compute_units);

/* Attention forward that fills the last, partial round of workgroups (asynchronous; one kernel,
 * plus a small combine pass when it cuts tiles). The same operation as lsv_attn_fwd (the varlen
 * forward of FastVideo #2049). The query tiles of the whole rounds run as in lsv_attn_fwd, on
 * the same XCDs and in the same order; each XCD's tiles of its last, partial round are cut into
 * key ranges (lsv_attn_fwd_tail_plan) that run after them on that XCD, and their partial
 * softmaxes are merged as in lsv_attn_fwd_split:
 *     LSE = ln sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r   (fp32, then bf16 nearest even).
 * A launch of n query tiles otherwise runs ceil(n / compute_units) rounds with the last one
 * partly idle: 14 heads x 19,394 tokens is 1,064 tiles, 4.16 rounds of 256 compute units. Results differ from lsv_attn_fwd's by rounding only (the whole
 * tiles are bit-identical to it) and are deterministic. When nothing is cut this is
 * lsv_attn_fwd itself and the workspace is not used.
 *
 * q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
 * stream: as for lsv_attn_fwd (same layouts, limits and skipped-segment rule).
 * compute_units  workgroup slots to plan for: a positive multiple of 8 (the device's compute-unit
 *              count), else LSV_ERR_INVALID_ARG.
 * workspace    device pointer, 16-byte aligned, at least n_tail_tiles * n_split * 256 * 129 * 4
 *              bytes for the plan (lsv_attn_fwd_tail_workspace_size always suffices); overwritten.
 *              Owned by the caller.
 */
int lsv_attn_fwd_tail(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens,
                      int32_t n_seqs, int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim,
                      float scale, int32_t compute_units, void* workspace, int64_t workspace_bytes, void* stream);

/* FP8 (e4m3) attention forward on the caller's stream (asynchronous).
 *
 * The operation (TensorRT-LLM PR #21275, the MiniMax-H3 recipe commit: attention with
 * --qk-dtype fp8 --v-dtype fp8 and per-tensor FP8 descales, the LSE returned; over the varlen
 * forward of FastVideo #2049): q, k, v hold OCP FP8 e4m3 bytes (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities) whose real values are descale_x * x8; then, as for
 * lsv_attn_fwd,
 *     z_ij = scale * (descale_q q8_i) . (descale_k k8_j),   O_i = sum_j softmax_j(z_ij) descale_v v8_j,
 *     LSE_i = ln sum_j exp(z_ij).
 * The attention weights are rounded to e4m3 for the P.V product and O is normalised by the sum
 * of those rounded weights; the LSE uses the fp32 weights. O is bf16, LSE fp32.
 *
 * q, k, v      device pointers, uint8 e4m3 [total_tokens, n_heads, head_dim], 16-byte aligned.
 * descale_q, descale_k, descale_v  finite, > 0.
 * o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale, stream:
 *              as for lsv_attn_fwd (same layouts, limits and skipped-segment rule; the 32-bit
 *              offset limit is max_seqlen * n_heads * head_dim + head_dim < 2^32 bytes).
 */
int lsv_attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k, float descale_v,
                     void* o, float* lse, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                     int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale, void* stream);

/* FP8 (e4m3) attention forward that fills the last, partial round of workgroups (asynchronous;
 * one kernel, plus a small combine pass when it cuts tiles): the operation of lsv_attn_fwd_fp8,
 * launched as lsv_attn_fwd_tail launches the BF16 forward. The query tiles of the whole rounds
 * run as in lsv_attn_fwd_fp8 (bit-identical rows); each XCD's tiles of its last, partial round are
 * cut into the key ranges of lsv_attn_fwd_tail_plan (the same plan: FP8 query tiles are also 256
 * rows), each range's dequantised, normalised O kept in fp32 with its LSE, and merged per row:
 *     LSE = ln sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r   (fp32, then bf16 nearest even).
 * Each range rounds its own weights to e4m3 against its own running max, so the cut rows differ
 * from lsv_attn_fwd_fp8's by rounding only; deterministic. When nothing is cut this is
 * lsv_attn_fwd_fp8 itself and the workspace is not used.
 *
 * q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens,
 * n_heads, head_dim, scale, stream: as for lsv_attn_fwd_fp8.
 * compute_units, workspace, workspace_bytes: as for lsv_attn_fwd_tail
 *              (lsv_attn_fwd_tail_workspace_size(compute_units) bytes always suffice).
 */
int lsv_attn_fwd_fp8_tail(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                          float descale_v, void* o, float* lse, const int32_t* cu_seqlens, int32_t n_seqs,
                          int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale,
                          int32_t compute_units, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes lsv_attn_bwd needs: two fp32 values per (head, token), i.e.
 * 8 * total_tokens * n_heads. Returns -1 for a negative size or n_heads < 1. */
int64_t lsv_attn_bwd_workspace_size(int64_t total_tokens, int32_t n_heads);

/* Attention backward on the caller's stream (asynchronous; two kernels -- a statistics pass,
 * then the dK/dV and dQ passes in one launch -- and no atomics: the same inputs give
 * bit-identical gradients on every run).
 *
 * The operation (FastVideo #2049, diff of fastvideo/attention/utils/flash_attn_cute.py, the
 * varlen backward op: it takes q, k, v, out, dout, lse, the softmax scale, causal=False and
 * the forward's cu_seqlens / max_seqlen, and returns dq, dk, dv shaped like q, k, v; the
 * page's test fakes pin that argument list). For every segment, head, query i and key j of
 * the segment, with P_ij = exp(scale q_i.k_j - LSE_i):
 *     D_i   = dO_i . O_i
 *     dS_ij = P_ij (dO_i . v_j - D_i)
 *     dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
 * P is computed in fp32 from the given fp32 LSE; P (for dV) and dS (for dQ, dK) are rounded
 * to bf16 for the matrix products, which accumulate in fp32; the gradients are rounded to
 * bf16 (nearest even).
 *
 * q, k, v, o, dout  device pointers, bf16 [total_tokens, n_heads, head_dim], 16-byte aligned;
 *              o and lse are the forward's outputs for these q, k, v (lsv_attn_fwd).
 * lse          device pointer, fp32 [n_heads, total_tokens].
 * dq, dk, dv   device pointers, bf16, same layout as q, 16-byte aligned. Written for every
 *              token row inside a segment; other rows untouched.
 * cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale: as for
 *              lsv_attn_fwd (same limits and the same skipped-segment rule).
 * workspace    device pointer, 4-byte aligned, at least lsv_attn_bwd_workspace_size bytes
 *              (else LSV_ERR_INVALID_ARG); overwritten. Owned by the caller.
 * stream       a hipStream_t, or NULL for the default stream.
 *
 * total_tokens * n_heads must stay below 2^31 (else LSV_ERR_UNSUPPORTED). Validation happens
 * before any HIP call; on error nothing is launched.
 */
int lsv_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs, int32_t max_seqlen,
                 int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale, void* workspace,
                 int64_t workspace_bytes, void* stream);

/* lsv_attn_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or training loops, harnesses that forbid
 * allocation). It computes exactly what lsv_attn_bwd computes, with the same kernels and
 * bit-identical gradients; the per-(head, token) statistics go to a scratch array that the
 * library holds in device memory, 2^27 bytes on each GPU it runs on, kept until the process ends.
 *
 * Arguments as for lsv_attn_bwd, without workspace / workspace_bytes. total_tokens * n_heads
 * must not exceed lsv_attn_bwd_noalloc_max_rows() (2^24, e.g. a 299,593-token segment at 56
 * heads), else LSV_ERR_UNSUPPORTED before any HIP call. The first call on a device looks up
 * that device's scratch address (a HIP runtime query, once per device); after that a call makes
 * no allocation and no synchronisation. The scratch is fully written by each call before it is
 * read, so nothing carries over from the previous call. Calls that overlap on one GPU (on
 * different streams, or from several threads without ordering) share the one scratch array and
 * race: order them on one stream.
 */
int lsv_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens, int32_t n_seqs,
                         int32_t max_seqlen, int64_t total_tokens, int32_t n_heads, int32_t head_dim, float scale,
                         void* stream);

/* The largest total_tokens * n_heads lsv_attn_bwd_noalloc accepts: 2^24. */
int64_t lsv_attn_bwd_noalloc_max_rows(void);

/* Fused QKV prologue on the caller's stream (asynchronous).
 *
 * The operation (FastVideo #2049, diff of
 * fastvideo/models/dits/minimax_h3_fusions/mk/qkv_prologue.py, module docstring and kernel;
 * MiniMaxH3Attention.forward on the same page rotates 96 of the 128 channels): every
 * (batch, position s, head) row x of Q, and of K with its own weight, becomes
 *     y_i   = x_i * rsqrt(mean_d x_d^2 + eps) * w_i
 *     out_i = y_i cos[s,i] - y_{i+R/2} sin[s,i]     for i < R/2
 *     out_i = y_i cos[s,i] + y_{i-R/2} sin[s,i]     for R/2 <= i < R
 *     out_i = y_i                                    for i >= R
 * computed in fp32 and rounded once to bf16 (nearest even); V is copied unchanged. The
 * three results are stacked [3, batch, seq_len, n_heads, head_dim] (plane 0 Q, 1 K, 2 V),
 * the layout the page's attention path consumes.
 *
 * q, k, v      device pointers, bf16 [batch, seq_len, n_heads, head_dim], 16-byte aligned.
 * q_weight, k_weight  device pointers, bf16 [head_dim] (the per-head norm weights).
 * cos, sin     device pointers, bf16 [seq_len, rotary_dim], 16-byte aligned; row s serves
 *              position s of every batch row and head. May be NULL when rotary_dim is 0.
 * out          device pointer, bf16 [3, batch, seq_len, n_heads, head_dim], 16-byte aligned,
 *              not overlapping any input. Fully written.
 * batch, seq_len  >= 0 (either 0: successful no-op); batch * seq_len * n_heads < 2^31.
 * n_heads      >= 1.
 * head_dim     must be 128.
 * rotary_dim   R: a multiple of 16 in [0, 128] (96 for the H3 blocks), else UNSUPPORTED.
 * eps          finite, >= 0 (1e-5 for the H3 blocks). With eps = 0 an all-zero row gives NaN.
 * stream       a hipStream_t, or NULL for the default stream.
 *
 * Validation happens before any HIP call; on error nothing is launched.
 */
int lsv_qkv_prologue(const void* q, const void* k, const void* v, const void* q_weight, const void* k_weight,
                     const void* cos, const void* sin, void* out, int64_t batch, int64_t seq_len, int32_t n_heads,
                     int32_t head_dim, int32_t rotary_dim, float eps, void* stream);

/* The QKV prologue's per-row step on one tensor (asynchronous): every (token t, head) row x of
 * x becomes y_i = x_i * rsqrt(mean_d x_d^2 + eps) * weight_i, rotated on its first R channels
 * with the cos/sin row of token t (as lsv_attn_fwd_qnorm describes), in fp32, rounded once to
 * bf16 (the MotionKernel qkv_prologue of FastVideo #2049; bit-identical to lsv_qkv_prologue's Q
 * or K plane for one sequence). The K side of a forward whose Q side is lsv_attn_fwd_qnorm.
 *
 * x, out       device pointers, bf16 [total_tokens, n_heads, head_dim], 16-byte aligned, not
 *              overlapping.
 * weight       device pointer, bf16 [head_dim].
 * cos, sin     device pointers, bf16 [total_tokens, rotary_dim], 16-byte aligned; may be NULL when
 *              rotary_dim is 0.
 * total_tokens >= 0 (0: successful no-op); total_tokens * n_heads < 2^31.
 * n_heads >= 1; head_dim must be 128; rotary_dim a multiple of 16 in [0, 128]; eps finite, >= 0.
 */
int lsv_norm_rope(const void* x, const void* weight, const void* cos, const void* sin, void* out,
                  int64_t total_tokens, int32_t n_heads, int32_t head_dim, int32_t rotary_dim, float eps,
                  void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* lsv_status_string(int status);

/* Dense BF16 MFMA peak of `device` in TFLOP/s at its reported maximum clock:
 * compute units x clock x 4096 flop per clock per compute unit (gfx950: one
 * 32x32x16 bf16 MFMA, 32768 flop, per 32 clocks on each of 4 SIMDs).
 * Writes *tflops and the CU count and clock (kHz) if the pointers are non-NULL. */
int lsv_device_peak(int device, double* tflops, int* compute_units, int* clock_khz);

/* Query-tile height (rows per workgroup) and key-tile width of the built kernel. */
int lsv_tile_config(int* block_q, int* block_k);

#ifdef __cplusplus
}
#endif

#endif /* LSV_H */
