"""Plain fp64 CPU oracle for the fused QKV prologue (per-head RMSNorm + partial RoPE).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
never imports, calls or links it, and it imports nothing from the product package.

What it computes (FastVideo #2049, diff of
``fastvideo/models/dits/minimax_h3_fusions/mk/qkv_prologue.py``, the module
docstring and the kernel body): for q, k, v of shape ``[B, S, H, D]``, every
(batch, position s, head) row ``x`` of Q and of K becomes::

    inv   = 1 / sqrt(mean_d x_d^2 + eps)
    y_d   = x_d * inv * w_d                               (w: that tensor's norm weight)
    out_i = y_i c_i - y_{i+R/2} s_i        for 0   <= i < R/2
    out_i = y_i c_i + y_{i-R/2} s_i        for R/2 <= i < R
    out_i = y_i                            for R   <= i < D

with ``c = cos[s, :]``, ``s = sin[s, :]`` (tables ``[S, R]``, indexed by the position
inside the sequence, shared by every batch row and head) and ``R`` the rotary width
(96 of 128 channels for MiniMax-H3: MiniMaxH3Attention.forward on the same page). V
is copied unchanged. The result is stacked ``[3 B, S, H, D]``: rotated Q, rotated K,
V (the kernel writes plane 0, 1, 2; the page's int32-plane test checks
``out[2B:] == v``). The kernel computes in fp32 and rounds once to bf16; this
oracle keeps the unrounded fp64 value.

Readings where the page is terse:
  * ``eps`` is the fp32 value handed to the kernel (1e-5 for the H3 blocks),
    widened exactly.
  * Tables and weights are bf16 (the page's wrapper casts cos/sin to the
    activation dtype; the norm weights are the module's bf16 parameters).
  * ``R`` is even; channels at and past ``R`` are normalised but not rotated.

Arithmetic: every input is a bf16 bit pattern widened exactly to fp64; all
steps are fp64 numpy, row by row, in the order written above.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64, f32_to_f64

__all__ = ["qkv_prologue_fp64", "norm_rope_rows_fp64"]


def norm_rope_rows_fp64(x_bits: np.ndarray, w_bits: np.ndarray, cos_bits: np.ndarray,
                        sin_bits: np.ndarray, eps: float):
    """RMSNorm + partial rotate-half RoPE of rows.

    Args:
      x_bits: uint16 ``[N, D]`` bf16 rows.
      w_bits: uint16 ``[D]`` bf16 norm weight.
      cos_bits, sin_bits: uint16 ``[N, R]`` bf16 table rows, one per input row.
      eps: the fp32 epsilon.

    Returns:
      ``(out, mag)`` fp64 ``[N, D]``: the exact result and, per element, the sum of
      the magnitudes of the terms added to form it (``|y_i c_i| + |partner s_i|``,
      or ``|y_i|`` for channels past ``R``), which bounds its floating-point
      cancellation.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    c = bf16_bits_to_f64(cos_bits)
    s = bf16_bits_to_f64(sin_bits)
    n, d = x.shape
    r = c.shape[1]
    if w.shape != (d,) or c.shape != (n, r) or s.shape != (n, r):
        raise ValueError("weight must be [D]; cos/sin must be [N, R]")
    if r % 2 or r > d:
        raise ValueError("rotary width must be even and at most head_dim")
    e = f32_to_f64(eps)
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=1) + e)     # 1 / sqrt(mean x^2 + eps)
    y = x * inv[:, None] * w[None, :]                   # normalised, weighted
    out = y.copy()                                      # channels >= R pass through
    mag = np.abs(y)
    h = r // 2
    if h:
        lo, hi = y[:, :h], y[:, h:r]
        out[:, :h] = lo * c[:, :h] - hi * s[:, :h]      # first half: partner i + R/2, -sin
        out[:, h:r] = hi * c[:, h:r] + lo * s[:, h:r]   # second half: partner i - R/2, +sin
        mag[:, :h] = np.abs(lo * c[:, :h]) + np.abs(hi * s[:, :h])
        mag[:, h:r] = np.abs(hi * c[:, h:r]) + np.abs(lo * s[:, h:r])
    return out, mag


def qkv_prologue_fp64(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                      q_weight_bits: np.ndarray, k_weight_bits: np.ndarray,
                      cos_bits: np.ndarray, sin_bits: np.ndarray, eps: float = 1e-5,
                      *, tokens=None):
    """Reference QKV prologue.

    Args:
      q_bits, k_bits, v_bits: uint16 ``[B, S, H, D]`` (or ``[S, H, D]``, i.e. B = 1).
      q_weight_bits, k_weight_bits: uint16 ``[D]``.
      cos_bits, sin_bits: uint16 ``[S, R]``.
      eps: fp32 epsilon.
      tokens: optional 1-D int array of flat token indices ``b * S + s`` to
        evaluate (default: all ``B * S``).

    Returns:
      dict with ``q``, ``k`` (fp64 ``[N, H, D]``), ``q_mag``, ``k_mag`` (the
      cancellation bounds, same shape), ``v`` (uint16 ``[N, H, D]``, the copy) and
      ``tokens`` (the N flat token indices).
    """
    if q_bits.ndim == 3:
        q_bits, k_bits, v_bits = q_bits[None], k_bits[None], v_bits[None]
    if q_bits.ndim != 4 or q_bits.shape != k_bits.shape or q_bits.shape != v_bits.shape:
        raise ValueError("q, k, v must share one [B, S, H, D] shape")
    b, s, h, d = q_bits.shape
    if cos_bits.shape != sin_bits.shape or cos_bits.ndim != 2 or cos_bits.shape[0] != s:
        raise ValueError("cos/sin must be [S, R] tables")
    tokens = np.arange(b * s, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pos = tokens % s
    qf = q_bits.reshape(b * s, h, d)[tokens]
    kf = k_bits.reshape(b * s, h, d)[tokens]
    cos_rows = np.repeat(cos_bits[pos], h, axis=0)      # one table row per (token, head) row
    sin_rows = np.repeat(sin_bits[pos], h, axis=0)
    q_out, q_mag = norm_rope_rows_fp64(qf.reshape(-1, d), q_weight_bits, cos_rows, sin_rows, eps)
    k_out, k_mag = norm_rope_rows_fp64(kf.reshape(-1, d), k_weight_bits, cos_rows, sin_rows, eps)
    n = len(tokens)
    return {
        "q": q_out.reshape(n, h, d), "k": k_out.reshape(n, h, d),
        "q_mag": q_mag.reshape(n, h, d), "k_mag": k_mag.reshape(n, h, d),
        "v": v_bits.reshape(b * s, h, d)[tokens].copy(), "tokens": tokens,
    }
