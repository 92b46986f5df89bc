"""Plain fp64 CPU oracle for the FP8 (e4m3) attention forward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path never
imports, calls or links it, and it imports nothing from the product package.

What it computes (TensorRT-LLM PR #21275, the MiniMax-H3 recipe commit: attention with
``--qk-dtype fp8 --v-dtype fp8``, per-tensor FP8 descales, the LSE returned; over the
varlen forward of FastVideo #2049): q, k, v are OCP FP8 e4m3 bytes ``[total, H, D]``
with fp32 per-tensor descales ``dq, dk, dv``. The real inputs are ``dq * q8``,
``dk * k8``, ``dv * v8``; for every segment ``[a, b)``, head and query ``i``::

    z_ij = sigma * (dq q8_i) . (dk k8_j)          j in [a, b)
    O_i  = sum_j softmax_j(z_ij) * dv v8_j
    LSE_i = max_j z_ij + ln sum_j exp(z_ij - max_j z_ij)

in fp64 from the exact byte values (the unrounded result; the kernel rounds its weights
to e4m3 and its output to bf16, which its error budget covers).

e4m3 (OCP 8-bit floating point, E4M3): sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import f32_to_f64, segments

__all__ = ["e4m3_bits_to_f64", "attention_fp8_fp64"]


def _decode_fields(bits) -> np.ndarray:
    """The format's definition, field by field."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


_TABLE = _decode_fields(np.arange(256, dtype=np.uint8))  # all 256 codes, by the definition


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """Exact value of e4m3 bytes (NaN for the two NaN codes): the definition, tabulated."""
    return _TABLE[np.asarray(bits, dtype=np.uint8)]


def attention_fp8_fp64(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, cu_seqlens,
                       scale: float, *, rows=None, workers: int | None = None):
    """Reference FP8 attention forward in fp64.

    Args:
      q8, k8, v8: uint8 ``[total, heads, head_dim]`` e4m3 bytes.
      descale_q, descale_k, descale_v, scale: fp32 values (widened exactly).
      cu_seqlens: ``[n_seqs + 1]`` segment boundaries starting at 0.
      rows: optional sorted token indices (default: every covered token).
      workers: threads over (segment, head) pairs; default: all usable cores.

    Returns:
      ``(out [R, H, D], lse [H, R], rows)``.
    """
    if q8.shape != k8.shape or q8.shape != v8.shape or q8.ndim != 3:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    total, n_heads, d = q8.shape
    segs = segments(cu_seqlens)
    if segs and segs[-1][1] > total:
        raise ValueError("cu_seqlens exceeds total_tokens")
    sigma = f32_to_f64(scale)
    dq, dk, dv = f32_to_f64(descale_q), f32_to_f64(descale_k), f32_to_f64(descale_v)
    if rows is None:
        rows = np.concatenate([np.arange(a, b, dtype=np.int64) for a, b in segs] or [np.zeros(0, np.int64)])
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), n_heads, d))
    lse = np.zeros((n_heads, len(rows)))
    covered = np.zeros(len(rows), bool)
    jobs = []
    for a, b in segs:
        lo, hi = np.searchsorted(rows, a), np.searchsorted(rows, b)
        if hi == lo:
            continue
        covered[lo:hi] = True
        jobs += [(a, b, h, lo, hi) for h in range(n_heads)]
    if not covered.all():
        raise ValueError("every requested row must lie inside a segment")

    def run(job):
        a, b, h, lo, hi = job
        idx = rows[lo:hi]
        qs = dq * e4m3_bits_to_f64(q8[idx, h])          # real query rows
        ks = dk * e4m3_bits_to_f64(k8[a:b, h])          # real keys of the segment
        vs = dv * e4m3_bits_to_f64(v8[a:b, h])
        z = sigma * (qs @ ks.T)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        l = e.sum(axis=1)
        out[lo:hi, h] = (e @ vs) / l[:, None]
        lse[h, lo:hi] = m + np.log(l)

    n = workers or len(os.sched_getaffinity(0))
    if n <= 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(n) as ex:
            list(ex.map(run, jobs))
    return out, lse, rows
