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
Blocks of rows only bound memory and spread the work over threads; no row's
arithmetic depends on which block it is in.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import bf16_bits_to_f64, f32_to_f64, segments

__all__ = ["attention_bwd_fp64"]

_ELEMS = 1 << 22   # score-matrix elements per block of rows (bounds the memory of one block)


def _block_rows(n_keys: int) -> int:
    """Rows per block of a segment with ``n_keys`` keys: at most 256, and few enough that one
    block's score matrix stays near ``_ELEMS`` elements."""
    return int(max(8, min(256, _ELEMS // max(n_keys, 1))))


class _Head:
    """One (segment, head): the bf16 inputs widened exactly to fp64, and the forward
    statistics of every query row of the segment (filled block by block)."""

    def __init__(self, q, k, v, do, a, b, h):
        self.a, self.b = a, b
        self.qs = bf16_bits_to_f64(q[a:b, h, :])
        self.ks = bf16_bits_to_f64(k[a:b, h, :])
        self.vs = bf16_bits_to_f64(v[a:b, h, :])
        self.dos = bf16_bits_to_f64(do[a:b, h, :])
        n = b - a
        self.lse = np.empty(n)
        self.dvec = np.empty(n)
        self.o = None


def _stats(hd, r0, r1, sigma, keep_o):
    """LSE_i and D_i = dO_i . O_i for query rows [r0, r1) of the segment (and O_i)."""
    z = (hd.qs[r0:r1] @ hd.ks.T) * sigma
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    o = (e @ hd.vs) / l[:, None]
    hd.lse[r0:r1] = m + np.log(l)
    hd.dvec[r0:r1] = np.sum(hd.dos[r0:r1] * o, axis=1)
    if keep_o:
        hd.o[r0:r1] = o


def _dq(hd, idx, sigma):
    """dQ_i for query rows ``idx`` (offsets in the segment)."""
    p = np.exp((hd.qs[idx] @ hd.ks.T) * sigma - hd.lse[idx, None])    # P_ij, j over the segment
    dp = hd.dos[idx] @ hd.vs.T                                         # dP_ij
    ds = p * (dp - hd.dvec[idx, None])                                 # dS_ij
    return sigma * (ds @ hd.ks)                                        # dQ_i


def _dkdv(hd, idx, sigma):
    """dK_j, dV_j for key rows ``idx`` (offsets in the segment)."""
    pt = np.exp((hd.ks[idx] @ hd.qs.T) * sigma - hd.lse[None, :])     # P_ij as [j, i]
    dpt = hd.vs[idx] @ hd.dos.T                                        # dP_ij as [j, i]
    dst = pt * (dpt - hd.dvec[None, :])                                # dS_ij as [j, i]
    return sigma * (dst @ hd.qs), pt @ hd.dos                          # dK_j, dV_j


def attention_bwd_fp64(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, do_bits: np.ndarray,
                       cu_seqlens, scale: float, *, q_rows=None, k_rows=None, workers: int | None = None,
                       return_forward: bool = False):
    """Reference attention backward in fp64.

    Args:
      q_bits, k_bits, v_bits, do_bits: uint16 ``[total_tokens, heads, head_dim]`` bf16.
      cu_seqlens: ``[n_seqs + 1]`` segment boundaries, starting at 0.
      scale: the softmax scale as passed to the kernel (rounded to fp32 here).
      q_rows / k_rows: optional sorted token indices for which to return ``dQ`` /
        ``dK, dV`` (each inside some segment); default: every covered token.
      workers: threads; default: all usable cores. Work is split into blocks of rows of
        one (segment, head), so a single long segment still uses every core.
      return_forward: also return the forward's fp64 ``O`` ``[total, H, D]`` and ``LSE``
        ``[H, total]`` of every segment that holds a requested row (zeros elsewhere).

    Returns:
      dict with ``dq`` ``[Rq, H, D]``, ``dk``, ``dv`` ``[Rk, H, D]`` (fp64) and the
      ``q_rows`` / ``k_rows`` they belong to (plus ``o``, ``lse`` with return_forward).
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
    q_cov = np.zeros(len(q_rows), bool)
    k_cov = np.zeros(len(k_rows), bool)
    heads = []          # (_Head, ql, qh, kl, kh)
    for a, b in segs:
        ql, qh = np.searchsorted(q_rows, a), np.searchsorted(q_rows, b)
        kl, kh = np.searchsorted(k_rows, a), np.searchsorted(k_rows, b)
        q_cov[ql:qh] = True
        k_cov[kl:kh] = True
        if qh > ql or kh > kl:
            for h in range(n_heads):
                heads.append((a, b, h, ql, qh, kl, kh))
    if not (q_cov.all() and k_cov.all()):
        raise ValueError("every requested row must lie inside a segment")
    out_o = np.zeros((total, n_heads, head_dim)) if return_forward else None
    out_lse = np.zeros((n_heads, total)) if return_forward else None

    n = workers or len(os.sched_getaffinity(0))
    pool = ThreadPoolExecutor(n) if n > 1 else None

    def run_all(fn, jobs):
        if pool is None:
            for j in jobs:
                fn(*j)
        else:
            list(pool.map(lambda j: fn(*j), jobs))

    def one_head(a, b, h, ql, qh, kl, kh):
        hd = _Head(q_bits, k_bits, v_bits, do_bits, a, b, h)
        if return_forward:
            hd.o = np.empty((b - a, head_dim))
        br = _block_rows(b - a)
        run_all(lambda r0: _stats(hd, r0, min(r0 + br, b - a), sigma, return_forward),
                [(r0,) for r0 in range(0, b - a, br)])

        def q_block(i0):
            i1 = min(i0 + br, qh - ql)
            dq[ql + i0:ql + i1, h] = _dq(hd, q_rows[ql + i0:ql + i1] - a, sigma)

        def k_block(i0):
            i1 = min(i0 + br, kh - kl)
            gk, gv = _dkdv(hd, k_rows[kl + i0:kl + i1] - a, sigma)
            dk[kl + i0:kl + i1, h] = gk
            dv[kl + i0:kl + i1, h] = gv

        run_all(q_block, [(i0,) for i0 in range(0, qh - ql, br)])
        run_all(k_block, [(i0,) for i0 in range(0, kh - kl, br)])
        if return_forward:
            out_o[a:b, h] = hd.o
            out_lse[h, a:b] = hd.lse

    try:
        if pool is None:
            for job in heads:
                one_head(*job)
        else:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1, user_api="blas"):
                for job in heads:
                    one_head(*job)
    finally:
        if pool is not None:
            pool.shutdown()
    res = {"dq": dq, "dk": dk, "dv": dv, "q_rows": q_rows, "k_rows": k_rows}
    if return_forward:
        res["o"] = out_o
        res["lse"] = out_lse
    return res
