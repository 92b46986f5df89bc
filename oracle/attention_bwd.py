"""Plain fp64 CPU oracle for the backward of the dense non-causal varlen attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
never imports, calls or links it, and it imports nothing from the product package.

What it computes: the gradients of ``L = sum(dO * O)`` for the forward that
``attention.py`` defines (FastVideo #2049, diff of
``fastvideo/attention/utils/flash_attn_cute.py``: the varlen backward op takes
``q, k, v, out, dout, lse``, the softmax scale, ``causal=False`` and the same
``cu_seqlens`` / ``max_seqlen`` as the forward, and returns ``dq, dk, dv`` shaped
like ``q, k, v``; the page's test fakes pin that argument list). Per segment
``[a, b)``, head ``h``, query ``i`` and key ``j`` of the segment::

    P_ij  = exp(sigma q_i . k_j - LSE_i)          (the forward's softmax)
    O_i   = sum_j P_ij v_j
    D_i   = dO_i . O_i
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = sigma sum_j dS_ij k_j
    dK_j  = sigma sum_i dS_ij q_i
    dV_j  = sum_i P_ij dO_i

This is the chain rule through ``O = softmax(sigma Q K^T) V`` written out (the
softmax Jacobian ``diag(P) - P P^T`` gives ``dS = P * (dP - rowsum(P * dP))``, and
``rowsum(P * dP) = dO . O``). The oracle uses the exact fp64 ``O`` and ``LSE`` of
the same inputs, i.e. it differentiates the exact function; the kernel is handed
the bf16 ``O`` and fp32 ``LSE`` of a forward pass, and that rounding is part of
its error budget.

Arithmetic: bf16 inputs widened exactly to fp64; per (segment, head) the
forward statistics (``LSE``, ``O``, ``D``) are computed for every query of the
segment in blocks of rows; then every requested output row is its own sum
above (a query row for ``dQ``, a key row for ``dK``/``dV``), with numpy matmuls.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import bf16_bits_to_f64, f32_to_f64, segments

__all__ = ["attention_bwd_fp64"]

_BLOCK = 256


def _stats(qs, ks, vs, dos, sigma):
    """LSE and D for every query row of one (segment, head)."""
    n = qs.shape[0]
    lse = np.empty(n)
    dvec = np.empty(n)
    for r0 in range(0, n, _BLOCK):
        z = (qs[r0:r0 + _BLOCK] @ ks.T) * sigma
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        l = e.sum(axis=1)
        o = (e @ vs) / l[:, None]
        lse[r0:r0 + _BLOCK] = m + np.log(l)
        dvec[r0:r0 + _BLOCK] = np.sum(dos[r0:r0 + _BLOCK] * o, axis=1)    # D_i = dO_i . O_i
    return lse, dvec


def _one(q, k, v, do, a, b, h, q_rows, k_rows, sigma):
    qs = bf16_bits_to_f64(q[a:b, h, :])
    ks = bf16_bits_to_f64(k[a:b, h, :])
    vs = bf16_bits_to_f64(v[a:b, h, :])
    dos = bf16_bits_to_f64(do[a:b, h, :])
    lse, dvec = _stats(qs, ks, vs, dos, sigma)
    d = qs.shape[1]
    dq = np.empty((len(q_rows), d))
    for r0 in range(0, len(q_rows), _BLOCK):
        idx = q_rows[r0:r0 + _BLOCK] - a
        p = np.exp((qs[idx] @ ks.T) * sigma - lse[idx, None])     # P_ij, j over the segment
        dp = dos[idx] @ vs.T                                      # dP_ij
        ds = p * (dp - dvec[idx, None])                           # dS_ij
        dq[r0:r0 + _BLOCK] = sigma * (ds @ ks)                    # dQ_i
    dk = np.empty((len(k_rows), d))
    dv = np.empty((len(k_rows), d))
    for c0 in range(0, len(k_rows), _BLOCK):
        idx = k_rows[c0:c0 + _BLOCK] - a
        pt = np.exp((ks[idx] @ qs.T) * sigma - lse[None, :])      # P_ij as [j, i]
        dpt = vs[idx] @ dos.T                                     # dP_ij as [j, i]
        dst = pt * (dpt - dvec[None, :])                          # dS_ij as [j, i]
        dv[c0:c0 + _BLOCK] = pt @ dos                             # dV_j
        dk[c0:c0 + _BLOCK] = sigma * (dst @ qs)                   # dK_j
    return dq, dk, dv


def attention_bwd_fp64(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, do_bits: np.ndarray,
                       cu_seqlens, scale: float, *, q_rows=None, k_rows=None, workers: int | None = None):
    """Reference attention backward in fp64.

    Args:
      q_bits, k_bits, v_bits, do_bits: uint16 ``[total_tokens, heads, head_dim]`` bf16.
      cu_seqlens: ``[n_seqs + 1]`` segment boundaries, starting at 0.
      scale: the softmax scale as passed to the kernel (rounded to fp32 here).
      q_rows / k_rows: optional sorted token indices for which to return ``dQ`` /
        ``dK, dV`` (each inside some segment); default: every covered token.
      workers: threads over (segment, head) pairs; default: all usable cores.

    Returns:
      dict with ``dq`` ``[Rq, H, D]``, ``dk``, ``dv`` ``[Rk, H, D]`` (fp64) and the
      ``q_rows`` / ``k_rows`` they belong to.
    """
    if not (q_bits.shape == k_bits.shape == v_bits.shape == do_bits.shape) or q_bits.ndim != 3:
        raise ValueError("q, k, v, do must share one [total_tokens, heads, head_dim] shape")
    total, n_heads, head_dim = q_bits.shape
    segs = segments(cu_seqlens)
    if segs and segs[-1][1] > total:
        raise ValueError("cu_seqlens exceeds total_tokens")
    sigma = f32_to_f64(scale)
    every = np.concatenate([np.arange(a, b, dtype=np.int64) for a, b in segs] or [np.zeros(0, np.int64)])
    q_rows = every if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_rows = every if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((len(q_rows), n_heads, head_dim))
    dk = np.zeros((len(k_rows), n_heads, head_dim))
    dv = np.zeros((len(k_rows), n_heads, head_dim))
    jobs = []
    q_cov = np.zeros(len(q_rows), bool)
    k_cov = np.zeros(len(k_rows), bool)
    for a, b in segs:
        ql, qh = np.searchsorted(q_rows, a), np.searchsorted(q_rows, b)
        kl, kh = np.searchsorted(k_rows, a), np.searchsorted(k_rows, b)
        q_cov[ql:qh] = True
        k_cov[kl:kh] = True
        if qh > ql or kh > kl:
            for h in range(n_heads):
                jobs.append((a, b, h, ql, qh, kl, kh))
    if not (q_cov.all() and k_cov.all()):
        raise ValueError("every requested row must lie inside a segment")

    def run(job):
        a, b, h, ql, qh, kl, kh = job
        gq, gk, gv = _one(q_bits, k_bits, v_bits, do_bits, a, b, h, q_rows[ql:qh], k_rows[kl:kh], sigma)
        dq[ql:qh, h] = gq
        dk[kl:kh, h] = gk
        dv[kl:kh, h] = gv

    n = workers or len(os.sched_getaffinity(0))
    if n <= 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(n) as ex:
            list(ex.map(run, jobs))
    return {"dq": dq, "dk": dk, "dv": dv, "q_rows": q_rows, "k_rows": k_rows}
