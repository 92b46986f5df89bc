"""Plain fp64 CPU oracle for the dense non-causal varlen attention forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product package.

What it computes (the plain definition, not the online algorithm):

For every packed segment ``[a, b) = [cu_seqlens[s], cu_seqlens[s+1])``, every
head ``h`` and every query row ``i`` in ``[a, b)``::

    z_ij     = sigma * sum_d q[i,h,d] * k[j,h,d]        for j in [a, b) only
    m_i      = max_j z_ij
    l_i      = sum_j exp(z_ij - m_i)
    O[i,h,:] = sum_j exp(z_ij - m_i) * v[j,h,:] / l_i
    LSE[h,i] = m_i + ln(l_i)

Sources (the pages):
  * FastVideo #2049 "FA4 JIT cache vs tuning env, MXFP8 import and scale dtype,
    H3 VSA gate double quantization", diff of
    ``fastvideo/attention/utils/flash_attn_cute.py``: the varlen forward takes
    q/k/v packed as ``[total_tokens, heads, head_dim]`` with one
    ``cu_seqlens`` int32 vector used for both queries and keys, an explicit
    ``softmax_scale``, ``causal=False`` for these blocks, ``num_splits=1`` and
    ``return_lse=True``; it returns ``(out, lse)``, and returns early on empty
    input.
  * Same page, test ``test_flash_attn_cute_varlen_kwargs.py``: for q of shape
    ``[7, 2, 8]`` with ``cu_seqlens = [0, 7]`` and ``softmax_scale = 0.125``
    the output has shape ``[7, 2, 8]`` and the LSE has shape ``[2, 7]``, i.e.
    LSE is laid out ``[heads, total_tokens]``.
  * TensorRT-LLM PR #21275 "Request FA4's 2-CTA kernel for MiniMax-H3 on SM103
    and SM107", Description: the transformer blocks run non-causal BF16
    attention at the packed clip length (19k to 104k tokens, 56 heads x 128).

Readings where the pages are silent:
  * LSE is the natural log of the sum of exponentials of the *scaled* logits
    (the FlashAttention convention); the pages never state the base.
  * ``sigma`` is the fp32 value handed to the kernel, widened exactly to fp64.
  * Rows not covered by any segment are not part of any output row set.

Arithmetic: inputs are bf16 bit patterns (uint16); each is widened exactly to
fp64. Products of two bf16 values are exact in fp64. Everything else is fp64
numpy (``matmul``, ``exp``, ``log``, ``max``, ``sum``) evaluated row by row:
rows are independent in the definition, so this module groups query rows into
blocks only to bound memory; no arithmetic is reordered or fused beyond the
definition above.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["bf16_bits_to_f64", "f32_to_f64", "attention_fp64", "segments"]

_ROW_BLOCK = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64.

    A bf16 value is the upper half of an IEEE binary32 word, so ``bits << 16``
    reinterpreted as float32 is the exact value; float32 -> float64 is exact.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_f64(x: float) -> float:
    """The fp32 value nearest ``x`` (round to nearest even), widened to fp64."""
    return float(np.float64(np.float32(x)))


def segments(cu_seqlens) -> list[tuple[int, int]]:
    """``[(a, b)]`` for every segment, from the cumulative ``cu_seqlens`` vector."""
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) == 0 or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    for x, y in zip(cu[:-1], cu[1:]):
        if y < x:
            raise ValueError("cu_seqlens must be non-decreasing")
    return list(zip(cu[:-1], cu[1:]))


def _head_rows(q, k, v, a, b, h, rows, sigma):
    """O and LSE of query ``rows`` (absolute token indices in [a, b)) of one head."""
    ks = bf16_bits_to_f64(k[a:b, h, :])          # [L, D]
    vs = bf16_bits_to_f64(v[a:b, h, :])          # [L, D]
    out = np.empty((len(rows), ks.shape[1]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    for r0 in range(0, len(rows), _ROW_BLOCK):
        idx = rows[r0:r0 + _ROW_BLOCK]
        qb = bf16_bits_to_f64(q[idx, h, :])      # [R, D]
        z = (qb @ ks.T) * sigma                  # z_ij = sigma * sum_d q_id k_jd
        m = z.max(axis=1)                        # m_i
        e = np.exp(z - m[:, None])               # exp(z_ij - m_i)
        l = e.sum(axis=1)                        # l_i
        out[r0:r0 + len(idx)] = (e @ vs) / l[:, None]
        lse[r0:r0 + len(idx)] = m + np.log(l)
    return out, lse


def attention_fp64(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                   cu_seqlens, scale: float, *, rows=None, workers: int | None = None):
    """Reference attention forward in fp64.

    Args:
      q_bits, k_bits, v_bits: uint16 arrays ``[total_tokens, heads, head_dim]``
        holding bf16 bit patterns.
      cu_seqlens: cumulative segment boundaries, ``[n_seqs + 1]``, starting at 0.
      scale: the softmax scale as passed to the kernel (rounded to fp32 here).
      rows: optional sorted 1-D array of absolute query token indices to
        evaluate (every index must lie inside some segment). ``None`` means every
        token covered by a segment.
      workers: threads over (segment, head) pairs; default: all usable cores.

    Returns:
      ``(out, lse, rows)``: ``out`` fp64 ``[R, heads, head_dim]``, ``lse`` fp64
      ``[heads, R]`` (natural log) and the int64 row indices ``R`` they belong to.
    """
    if q_bits.shape != k_bits.shape or q_bits.shape != v_bits.shape or q_bits.ndim != 3:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    total, n_heads, head_dim = q_bits.shape
    segs = segments(cu_seqlens)
    if segs and segs[-1][1] > total:
        raise ValueError("cu_seqlens exceeds total_tokens")
    sigma = f32_to_f64(scale)
    if rows is None:
        rows = np.concatenate([np.arange(a, b, dtype=np.int64) for a, b in segs] or
                              [np.zeros(0, dtype=np.int64)])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), n_heads, head_dim), dtype=np.float64)
    lse = np.zeros((n_heads, len(rows)), dtype=np.float64)
    covered = np.zeros(len(rows), dtype=bool)

    jobs = []
    for a, b in segs:
        lo, hi = np.searchsorted(rows, a, "left"), np.searchsorted(rows, b, "left")
        if hi > lo:
            covered[lo:hi] = True
            for h in range(n_heads):
                jobs.append((a, b, h, lo, hi))
    if not covered.all():
        raise ValueError("every requested row must lie inside a segment")

    def run(job):
        a, b, h, lo, hi = job
        o, s = _head_rows(q_bits, k_bits, v_bits, a, b, h, rows[lo:hi], sigma)
        out[lo:hi, h, :] = o
        lse[h, lo:hi] = s

    n = workers or len(os.sched_getaffinity(0))
    if n <= 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(n) as ex:
            list(ex.map(run, jobs))
    return out, lse, rows
