"""lsv: dense non-causal varlen attention for MI355X (gfx950): the BF16 forward, its
deterministic backward, an FP8 (e4m3) forward, and the fused QKV prologue (QK RMSNorm +
partial RoPE) that feeds them.

Thin ctypes binding over the C ABI in ``include/lsv.h`` (``liblsv.so``, built in-tree by
``python -m long_sequence_video_amd.build``). The functions named like the C entry points
(``lsv_attn_fwd``, ``lsv_attn_fwd_split``, ``lsv_attn_fwd_split_workspace_size``, ``lsv_attn_fwd_fp8``,
``lsv_attn_bwd``, ``lsv_attn_bwd_workspace_size``, ``lsv_attn_bwd_noalloc``,
``lsv_attn_bwd_noalloc_max_rows``, ``lsv_qkv_prologue``, ``lsv_attn_fwd_qnorm``, ``lsv_norm_rope``,
``lsv_attn_fwd_tail``, ``lsv_attn_fwd_tail_plan``, ``lsv_attn_fwd_tail_workspace_size``,
``lsv_attn_fwd_fp8_tail``, ``lsv_attn_fwd_qnorm_tail``, ``lsv_status_string``, ``lsv_device_peak``, ``lsv_tile_config``) only marshal arguments;
``attn_fwd``, ``attn_fwd_split``, ``attn_fwd_tail``, ``attn_fwd_fp8``, ``attn_fwd_fp8_tail``, ``attn_bwd``,
``attn_bwd_noalloc``, ``qkv_prologue``, ``attn_fwd_qnorm`` (and its ``compute_units`` form) and ``norm_rope`` add torch-tensor conveniences (shape checks, output and workspace allocation, the current
stream). There is no fallback: if the library is missing or a call fails, an exception is
raised.

Buffers these conveniences allocate come from torch's caching allocator on the current
stream; when the work runs on another ``stream``, each is marked as in use by that stream
(``record_stream``), so the allocator does not hand it out again before the kernels are done.
When ``max_seqlen`` is omitted it is computed from ``cu_seqlens`` with a device-to-host copy,
which synchronises; the C library itself never reads ``cu_seqlens`` on the host.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH", "LsvError", "load_library", "lsv_attn_fwd", "lsv_attn_fwd_split", "lsv_attn_fwd_split_workspace_size",
    "lsv_attn_fwd_fp8", "attn_fwd_fp8", "lsv_attn_bwd", "lsv_attn_bwd_workspace_size", "lsv_attn_bwd_noalloc",
    "lsv_attn_bwd_noalloc_max_rows", "attn_bwd_noalloc", "lsv_qkv_prologue", "lsv_attn_fwd_qnorm", "lsv_norm_rope",
    "attn_fwd_qnorm", "norm_rope", "lsv_attn_fwd_tail", "lsv_attn_fwd_tail_plan", "lsv_attn_fwd_tail_workspace_size",
    "attn_fwd_tail", "lsv_attn_fwd_fp8_tail", "attn_fwd_fp8_tail", "lsv_attn_fwd_qnorm_tail",
    "lsv_status_string", "lsv_device_peak", "lsv_tile_config", "attn_fwd", "attn_fwd_split", "choose_split",
    "attn_bwd", "qkv_prologue", "flops", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsv.so")
EXPORTED_SYMBOLS = ("lsv_attn_fwd", "lsv_attn_fwd_split", "lsv_attn_fwd_split_workspace_size", "lsv_attn_fwd_fp8",
                    "lsv_attn_bwd", "lsv_attn_bwd_workspace_size", "lsv_attn_bwd_noalloc",
                    "lsv_attn_bwd_noalloc_max_rows", "lsv_qkv_prologue", "lsv_attn_fwd_qnorm", "lsv_norm_rope",
                    "lsv_attn_fwd_tail", "lsv_attn_fwd_tail_plan", "lsv_attn_fwd_tail_workspace_size",
                    "lsv_attn_fwd_fp8_tail", "lsv_attn_fwd_qnorm_tail", "lsv_status_string", "lsv_device_peak",
                    "lsv_tile_config")

LSV_OK = 0
LSV_ERR_INVALID_ARG = -1
LSV_ERR_UNSUPPORTED = -2
LSV_ERR_ALIGNMENT = -3
LSV_ERR_LAUNCH = -4
LSV_ERR_HIP = -5

_lib = None


class LsvError(ValueError):
    """A negative status returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lsv_status_string(status)} (status {status})")


def _keep_for(stream, *tensors) -> None:
    """Mark tensors this binding allocated as in use by ``stream`` when the kernels run there
    rather than on the current stream (torch's allocator then waits for that stream's work
    before reusing their memory)."""
    import torch
    if stream != torch.cuda.current_stream(stream.device):
        for t in tensors:
            if t is not None:
                t.record_stream(stream)


def load_library(path: str = LIB_PATH):
    """Load ``liblsv.so`` (once) and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m long_sequence_video_amd.build`")
    # torch ships its own HIP runtime. Loaded first, it also serves this library (same soname);
    # loaded after it, the library would have mapped the system's copy as well, and the two
    # runtimes in one process do not share devices, streams or memory.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.lsv_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, ctypes.c_float, vp]
    lib.lsv_attn_fwd.restype = ctypes.c_int
    lib.lsv_attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, ctypes.c_float, i32, vp, i64,
                                       vp]
    lib.lsv_attn_fwd_split.restype = ctypes.c_int
    lib.lsv_attn_fwd_split_workspace_size.argtypes = [i64, i32, i32]
    lib.lsv_attn_fwd_split_workspace_size.restype = i64
    f = ctypes.c_float
    lib.lsv_attn_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, vp, i32, i32, i64, i32, i32, f, vp]
    lib.lsv_attn_fwd_fp8.restype = ctypes.c_int
    lib.lsv_attn_fwd_fp8_tail.argtypes = [vp, vp, vp, f, f, f, vp, vp, vp, i32, i32, i64, i32, i32, f, i32, vp, i64, vp]
    lib.lsv_attn_fwd_fp8_tail.restype = ctypes.c_int
    lib.lsv_attn_bwd.argtypes = [vp] * 10 + [i32, i32, i64, i32, i32, ctypes.c_float, vp, i64, vp]
    lib.lsv_attn_bwd.restype = ctypes.c_int
    lib.lsv_attn_bwd_workspace_size.argtypes = [i64, i32]
    lib.lsv_attn_bwd_workspace_size.restype = i64
    lib.lsv_attn_bwd_noalloc.argtypes = [vp] * 10 + [i32, i32, i64, i32, i32, ctypes.c_float, vp]
    lib.lsv_attn_bwd_noalloc.restype = ctypes.c_int
    lib.lsv_attn_bwd_noalloc_max_rows.argtypes = []
    lib.lsv_attn_bwd_noalloc_max_rows.restype = i64
    lib.lsv_qkv_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ctypes.c_float, vp]
    lib.lsv_qkv_prologue.restype = ctypes.c_int
    lib.lsv_attn_fwd_qnorm.argtypes = [vp] * 6 + [i32, ctypes.c_float, vp, vp, vp, i32, i32, i64, i32, i32,
                                       ctypes.c_float, vp]
    lib.lsv_attn_fwd_qnorm.restype = ctypes.c_int
    lib.lsv_attn_fwd_qnorm_tail.argtypes = [vp] * 6 + [i32, ctypes.c_float, vp, vp, vp, i32, i32, i64, i32, i32,
                                            ctypes.c_float, i32, vp, i64, vp]
    lib.lsv_attn_fwd_qnorm_tail.restype = ctypes.c_int
    lib.lsv_norm_rope.argtypes = [vp] * 5 + [i64, i32, i32, i32, ctypes.c_float, vp]
    lib.lsv_norm_rope.restype = ctypes.c_int
    lib.lsv_attn_fwd_tail.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, ctypes.c_float, i32, vp, i64,
                                      vp]
    lib.lsv_attn_fwd_tail.restype = ctypes.c_int
    lib.lsv_attn_fwd_tail_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.lsv_attn_fwd_tail_plan.restype = ctypes.c_int
    lib.lsv_attn_fwd_tail_workspace_size.argtypes = [i32]
    lib.lsv_attn_fwd_tail_workspace_size.restype = i64
    lib.lsv_status_string.argtypes = [ctypes.c_int]
    lib.lsv_status_string.restype = ctypes.c_char_p
    lib.lsv_device_peak.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(ctypes.c_int)]
    lib.lsv_device_peak.restype = ctypes.c_int
    lib.lsv_tile_config.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.lsv_tile_config.restype = ctypes.c_int
    _lib = lib
    return lib


def lsv_attn_fwd(q: int, k: int, v: int, o: int, lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int,
                 total_tokens: int, n_heads: int, head_dim: int, scale: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads,
                                       head_dim, scale, stream)


def lsv_attn_fwd_split(q: int, k: int, v: int, o: int, lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int,
                       total_tokens: int, n_heads: int, head_dim: int, scale: float, n_split: int, workspace: int,
                       workspace_bytes: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_split(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads,
                                             head_dim, scale, n_split, workspace, workspace_bytes, stream)


def lsv_attn_fwd_split_workspace_size(total_tokens: int, n_heads: int, n_split: int) -> int:
    return load_library().lsv_attn_fwd_split_workspace_size(total_tokens, n_heads, n_split)


def choose_split(seqlens, n_heads: int, compute_units: int = 256, max_split: int = 4,
                 min_range_keys: int = 8192) -> int:
    """The key split for ``attn_fwd_split`` (a host-side estimate from the segment lengths).

    The forward runs one 256-row query tile of one (segment, head) per workgroup and one
    workgroup per compute unit at a time; with n key ranges there are n times as many, shorter,
    workgroups, which fill the last round better but each pay a fixed start and epilogue and
    write fp32 partial rows that a second pass reads back. Measured on MI355X that pays only
    while a range of the longest segment keeps at least ``min_range_keys`` keys (19,394 x 14:
    2.53 -> 2.47 ms with 2 ranges; 4,096 x 56: 0.47 -> 0.55 ms, slower). Returns 1 when the
    rounds are already at least 90% full, else the n in [2, max_split] with the fullest rounds
    among those whose ranges keep ``min_range_keys`` keys (the smallest n on ties).
    """
    lens = [int(s) for s in seqlens if int(s) > 0]
    if not lens:
        return 1
    units = sum((s + 255) // 256 for s in lens) * int(n_heads)

    def fill(n):
        work = units * n
        return work / (math.ceil(work / compute_units) * compute_units)

    if fill(1) >= 0.9:
        return 1
    best, best_fill = 1, fill(1)
    for n in range(2, max_split + 1):
        if max(lens) // n < min_range_keys:
            break
        if fill(n) > best_fill + 1e-9:
            best, best_fill = n, fill(n)
    return best


def lsv_attn_fwd_fp8(q: int, k: int, v: int, descale_q: float, descale_k: float, descale_v: float, o: int,
                     lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int, total_tokens: int, n_heads: int,
                     head_dim: int, scale: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_fp8(q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens, n_seqs,
                                           max_seqlen, total_tokens, n_heads, head_dim, scale, stream)


def lsv_attn_fwd_fp8_tail(q: int, k: int, v: int, descale_q: float, descale_k: float, descale_v: float, o: int,
                          lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int, total_tokens: int, n_heads: int,
                          head_dim: int, scale: float, compute_units: int, workspace: int, workspace_bytes: int,
                          stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_fp8_tail(q, k, v, descale_q, descale_k, descale_v, o, lse, cu_seqlens,
                                                n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                                                compute_units, workspace, workspace_bytes, stream)


def lsv_attn_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, cu_seqlens: int,
                 n_seqs: int, max_seqlen: int, total_tokens: int, n_heads: int, head_dim: int, scale: float,
                 workspace: int, workspace_bytes: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen,
                                       total_tokens, n_heads, head_dim, scale, workspace, workspace_bytes, stream)


def lsv_attn_bwd_workspace_size(total_tokens: int, n_heads: int) -> int:
    return load_library().lsv_attn_bwd_workspace_size(total_tokens, n_heads)


def lsv_attn_bwd_noalloc(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
                         cu_seqlens: int, n_seqs: int, max_seqlen: int, total_tokens: int, n_heads: int,
                         head_dim: int, scale: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, n_seqs, max_seqlen,
                                               total_tokens, n_heads, head_dim, scale, stream)


def lsv_attn_bwd_noalloc_max_rows() -> int:
    """The largest ``total_tokens * n_heads`` that ``lsv_attn_bwd_noalloc`` accepts."""
    return load_library().lsv_attn_bwd_noalloc_max_rows()


def lsv_qkv_prologue(q: int, k: int, v: int, q_weight: int, k_weight: int, cos: int, sin: int, out: int,
                     batch: int, seq_len: int, n_heads: int, head_dim: int, rotary_dim: int, eps: float,
                     stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_qkv_prologue(q, k, v, q_weight, k_weight, cos, sin, out, batch, seq_len, n_heads,
                                           head_dim, rotary_dim, eps, stream)


def lsv_attn_fwd_qnorm(q: int, k: int, v: int, q_weight: int, cos: int, sin: int, rotary_dim: int, eps: float,
                       o: int, lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int, total_tokens: int,
                       n_heads: int, head_dim: int, scale: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_qnorm(q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens,
                                             n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale, stream)


def lsv_attn_fwd_qnorm_tail(q: int, k: int, v: int, q_weight: int, cos: int, sin: int, rotary_dim: int,
                            eps: float, o: int, lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int,
                            total_tokens: int, n_heads: int, head_dim: int, scale: float, compute_units: int,
                            workspace: int, workspace_bytes: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_qnorm_tail(q, k, v, q_weight, cos, sin, rotary_dim, eps, o, lse, cu_seqlens,
                                                  n_seqs, max_seqlen, total_tokens, n_heads, head_dim, scale,
                                                  compute_units, workspace, workspace_bytes, stream)


def lsv_norm_rope(x: int, weight: int, cos: int, sin: int, out: int, total_tokens: int, n_heads: int,
                  head_dim: int, rotary_dim: int, eps: float, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_norm_rope(x, weight, cos, sin, out, total_tokens, n_heads, head_dim, rotary_dim, eps,
                                        stream)


def lsv_attn_fwd_tail(q: int, k: int, v: int, o: int, lse: int, cu_seqlens: int, n_seqs: int, max_seqlen: int,
                      total_tokens: int, n_heads: int, head_dim: int, scale: float, compute_units: int, workspace: int,
                      workspace_bytes: int, stream: int | None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return load_library().lsv_attn_fwd_tail(q, k, v, o, lse, cu_seqlens, n_seqs, max_seqlen, total_tokens, n_heads,
                                            head_dim, scale, compute_units, workspace, workspace_bytes, stream)


def lsv_attn_fwd_tail_plan(n_seqs: int, max_seqlen: int, n_heads: int, compute_units: int) -> tuple[int, int]:
    """(key ranges per tail tile, tail tiles) of lsv_attn_fwd_tail for these sizes."""
    s, t = ctypes.c_int32(), ctypes.c_int64()
    rc = load_library().lsv_attn_fwd_tail_plan(n_seqs, max_seqlen, n_heads, compute_units, ctypes.byref(s),
                                               ctypes.byref(t))
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_tail_plan")
    return s.value, t.value


def lsv_attn_fwd_tail_workspace_size(compute_units: int) -> int:
    return load_library().lsv_attn_fwd_tail_workspace_size(compute_units)


def lsv_status_string(status: int) -> str:
    return load_library().lsv_status_string(status).decode()


def lsv_device_peak(device: int = 0) -> tuple[float, int, int]:
    """(dense BF16 MFMA TFLOP/s at the reported max clock, compute units, clock kHz)."""
    tf, cus, khz = ctypes.c_double(), ctypes.c_int(), ctypes.c_int()
    rc = load_library().lsv_device_peak(device, ctypes.byref(tf), ctypes.byref(cus), ctypes.byref(khz))
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_device_peak")
    return tf.value, cus.value, khz.value


def lsv_tile_config() -> tuple[int, int]:
    """(query rows per workgroup, keys per tile) of the built kernel."""
    bq, bk = ctypes.c_int(), ctypes.c_int()
    load_library().lsv_tile_config(ctypes.byref(bq), ctypes.byref(bk))
    return bq.value, bk.value


def flops(seqlens, n_heads: int, head_dim: int = 128) -> float:
    """Attention forward flops counted as sum over sequences of 4 * S^2 * H * D."""
    return float(sum(4.0 * s * s * n_heads * head_dim for s in seqlens))


def attn_fwd(q, k, v, cu_seqlens, max_seqlen: int | None = None, scale: float | None = None, *, out=None,
             lse=None, stream=None):
    """Attention forward on torch tensors (all on one GPU).

    Args:
      q, k, v: bfloat16 ``[total_tokens, n_heads, 128]``, contiguous.
      cu_seqlens: int32 ``[n_seqs + 1]`` on the same device.
      max_seqlen: largest segment length; computed from ``cu_seqlens`` (a device-to-host
        copy) when omitted.
      scale: softmax scale; default ``1 / sqrt(head_dim)``.
      out, lse: optional preallocated outputs (``[T, H, D]`` bf16, ``[H, T]`` fp32).
      stream: a ``torch.cuda.Stream``; default: the current stream.

    Returns:
      ``(out, lse)``.
    """
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (k, v, cu_seqlens)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    if lse is None:
        lse = torch.empty((heads, total), dtype=torch.float32, device=dev)
        mine.append(lse)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    if out.device != dev or lse.device != dev:
        raise ValueError("out and lse must be on the same GPU as q")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, max_seqlen, total, heads, dim, scale,
                          s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd")
    return out, lse


def attn_fwd_split(q, k, v, cu_seqlens, max_seqlen: int | None = None, scale: float | None = None,
                   n_split: int = 2, *, out=None, lse=None, workspace=None, stream=None):
    """Attention forward with each segment's keys cut into ``n_split`` ranges (one GPU).

    Arguments as for ``attn_fwd``; ``workspace``, if given, is a contiguous device buffer of at
    least ``lsv_attn_fwd_split_workspace_size(total_tokens, heads, n_split)`` bytes (else one
    is allocated). Returns ``(out, lse)``.
    """
    import torch
    if n_split == 1:
        return attn_fwd(q, k, v, cu_seqlens, max_seqlen, scale, out=out, lse=lse, stream=stream)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (k, v, cu_seqlens)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    if lse is None:
        lse = torch.empty((heads, total), dtype=torch.float32, device=dev)
        mine.append(lse)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    if out.device != dev or lse.device != dev:
        raise ValueError("out and lse must be on the same GPU as q")
    need = lsv_attn_fwd_split_workspace_size(total, heads, n_split)
    if need < 0:
        raise ValueError("invalid sizes or n_split")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        mine.append(workspace)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same GPU")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, max_seqlen, total, heads, dim, scale,
                                n_split, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_split")
    return out, lse


def attn_fwd_tail(q, k, v, cu_seqlens, max_seqlen: int | None = None, scale: float | None = None, *,
                  compute_units: int | None = None, out=None, lse=None, workspace=None, stream=None):
    """Attention forward that cuts the query tiles of the last, partial round of workgroups into
    key ranges (``lsv_attn_fwd_tail``). Arguments as for ``attn_fwd``; ``compute_units`` defaults
    to the device's count; ``workspace``, if given, is a contiguous device buffer of at least
    ``lsv_attn_fwd_tail_workspace_size(compute_units)`` bytes (else one is allocated).
    Returns ``(out, lse)``."""
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (k, v, cu_seqlens)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    if compute_units is None:
        compute_units = lsv_device_peak(dev.index if dev.index is not None else torch.cuda.current_device())[1]
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    if lse is None:
        lse = torch.empty((heads, total), dtype=torch.float32, device=dev)
        mine.append(lse)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's GPU")
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev:
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor on q's GPU")
    need = lsv_attn_fwd_tail_workspace_size(compute_units)
    if need < 0:
        raise ValueError("compute_units must be a positive multiple of 8")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        mine.append(workspace)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same GPU")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_fwd_tail(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, max_seqlen, total, heads, dim, scale,
                               compute_units, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_tail")
    return out, lse


def qkv_prologue(q, k, v, q_weight, k_weight, cos, sin, *, eps: float = 1e-5, out=None, stream=None):
    """Fused QK RMSNorm + partial rotate-half RoPE, and the V copy, on torch tensors.

    Args:
      q, k, v: bfloat16 ``[B, S, H, 128]`` (or ``[S, H, 128]``), contiguous, one GPU.
      q_weight, k_weight: bfloat16 ``[128]``.
      cos, sin: bfloat16 ``[S, R]`` (R a multiple of 16, at most 128), or ``None`` for R = 0.
      eps: the RMSNorm epsilon (1e-5 for the H3 blocks).
      out: optional preallocated ``[3 B, S, H, 128]`` (``[3, S, H, 128]`` for 3-D inputs).
      stream: a ``torch.cuda.Stream``; default: the current stream.

    Returns:
      the stacked output: rotated Q, rotated K, V.
    """
    import torch
    if q.dim() not in (3, 4) or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, S, H, D] (or [S, H, D]) shape")
    tensors = [q, k, v, q_weight, k_weight] + ([cos, sin] if cos is not None else [])
    if any(t.dtype != torch.bfloat16 for t in tensors):
        raise ValueError("all inputs must be bfloat16")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("all inputs must be contiguous")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")
    b, s, h, d = (1, *q.shape) if q.dim() == 3 else tuple(q.shape)
    if (cos is None) != (sin is None):
        raise ValueError("cos and sin must both be given or both be None")
    rd = 0 if cos is None else int(cos.shape[-1])
    if cos is not None and (cos.shape != sin.shape or cos.dim() != 2 or cos.shape[0] != s):
        raise ValueError("cos/sin must be [S, R] tables")
    if q_weight.shape != (d,) or k_weight.shape != (d,):
        raise ValueError("norm weights must be [head_dim]")
    shape = (3, s, h, d) if q.dim() == 3 else (3 * b, s, h, d)
    mine = []
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        mine.append(out)
    if tuple(out.shape) != shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != dev:
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {shape}")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(st, *mine)
    with torch.cuda.device(dev):
        rc = lsv_qkv_prologue(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_weight.data_ptr(), k_weight.data_ptr(),
                              0 if cos is None else cos.data_ptr(), 0 if sin is None else sin.data_ptr(),
                              out.data_ptr(), b, s, h, d, rd, eps, st.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_qkv_prologue")
    return out


def _bwd_args(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, scale, dq, dk, dv):
    """Checks of the backward's torch arguments; returns (max_seqlen, scale, dq, dk, dv, the
    gradient tensors allocated here)."""
    import torch
    tensors = (q, k, v, out, dout)
    if any(t.dtype != torch.bfloat16 for t in tensors):
        raise ValueError("q, k, v, out, dout must be bfloat16")
    if q.dim() != 3 or any(t.shape != q.shape for t in tensors):
        raise ValueError("q, k, v, out, dout must share one [total_tokens, heads, head_dim] shape")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("q, k, v, out, dout must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (*tensors, lse, cu_seqlens)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q.shape
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    mine = []
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty_like(q)
            mine.append(g)
        if g.shape != q.shape or g.dtype != torch.bfloat16 or not g.is_contiguous() or g.device != dev:
            raise ValueError("dq, dk, dv must be contiguous bfloat16 tensors shaped like q")
        grads.append(g)
    return max_seqlen, scale, grads[0], grads[1], grads[2], mine


def attn_bwd(q, k, v, out, dout, lse, cu_seqlens, max_seqlen: int | None = None, scale: float | None = None, *,
             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward on torch tensors (all on one GPU).

    Args:
      q, k, v, out, dout: bfloat16 ``[total_tokens, n_heads, 128]``, contiguous (``out`` and
        ``lse`` from ``attn_fwd`` on the same q, k, v).
      lse: float32 ``[n_heads, total_tokens]``.
      cu_seqlens, max_seqlen, scale: as for ``attn_fwd``.
      dq, dk, dv: optional preallocated gradients (shaped like q).
      workspace: optional uint8 device buffer of at least ``lsv_attn_bwd_workspace_size`` bytes.
      stream: a ``torch.cuda.Stream``; default: the current stream.

    Returns:
      ``(dq, dk, dv)``.
    """
    import torch
    max_seqlen, scale, dq, dk, dv, mine = _bwd_args(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, scale, dq, dk,
                                                    dv)
    dev = q.device
    total, heads, dim = q.shape
    need = lsv_attn_bwd_workspace_size(total, heads)
    if need < 0:
        raise ValueError("invalid sizes")
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
        mine.append(workspace)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device buffer")
    ws_bytes = workspace.numel() * workspace.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                          max_seqlen, total, heads, dim, scale, workspace.data_ptr(), ws_bytes, s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, out, dout, lse, cu_seqlens, max_seqlen: int | None = None,
                     scale: float | None = None, *, dq=None, dk=None, dv=None, stream=None):
    """``attn_bwd`` through ``lsv_attn_bwd_noalloc``: the library's own device scratch holds
    the statistics, so nothing is allocated when ``dq``, ``dk`` and ``dv`` are given (and
    ``max_seqlen``, which otherwise costs a device-to-host copy). ``total_tokens * heads``
    must not exceed ``lsv_attn_bwd_noalloc_max_rows()``; calls that overlap on one GPU share
    the scratch and race. Arguments and result as for ``attn_bwd``."""
    import torch
    max_seqlen, scale, dq, dk, dv, mine = _bwd_args(q, k, v, out, dout, lse, cu_seqlens, max_seqlen, scale, dq, dk,
                                                    dv)
    dev = q.device
    total, heads, dim = q.shape
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                  lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens.data_ptr(),
                                  cu_seqlens.numel() - 1, max_seqlen, total, heads, dim, scale, s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_bwd_noalloc")
    return dq, dk, dv


def _tables(cos, sin, total, dev):
    """(rotary width, cos, sin) after checking per-token bf16 tables [total, R] (or both None)."""
    import torch
    if (cos is None) != (sin is None):
        raise ValueError("cos and sin must both be given or both be None")
    if cos is None:
        return 0, None, None
    for t in (cos, sin):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.shape[0] != total or not t.is_contiguous() or t.device != dev:
            raise ValueError("cos/sin must be contiguous bfloat16 [total_tokens, R] tables on the inputs' GPU")
    if cos.shape != sin.shape:
        raise ValueError("cos and sin must have one shape")
    return int(cos.shape[1]), cos, sin


def norm_rope(x, weight, cos=None, sin=None, *, eps: float = 1e-5, out=None, stream=None):
    """The QKV prologue's per-row RMSNorm + partial rotate-half RoPE on one tensor (e.g. K).

    Args:
      x: bfloat16 ``[total_tokens, heads, 128]``, contiguous, one GPU.
      weight: bfloat16 ``[128]``.
      cos, sin: bfloat16 ``[total_tokens, R]`` per-token tables (R a multiple of 16), or None.
      eps, out, stream: the epsilon, an optional preallocated output, the stream.

    Returns:
      the normalised, rotated tensor (bf16, shaped like x).
    """
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 3 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous bfloat16 [total_tokens, heads, head_dim] GPU tensor")
    dev = x.device
    total, heads, dim = x.shape
    if weight.dtype != torch.bfloat16 or weight.shape != (dim,) or not weight.is_contiguous() or weight.device != dev:
        raise ValueError("weight must be a contiguous bfloat16 [head_dim] tensor on x's GPU")
    rd, cos, sin = _tables(cos, sin, total, dev)
    mine = []
    if out is None:
        out = torch.empty_like(x)
        mine.append(out)
    if out.shape != x.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like x")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_norm_rope(x.data_ptr(), weight.data_ptr(), 0 if cos is None else cos.data_ptr(),
                           0 if sin is None else sin.data_ptr(), out.data_ptr(), total, heads, dim, rd, eps,
                           s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_norm_rope")
    return out


def attn_fwd_qnorm(q, k, v, q_weight, cos, sin, cu_seqlens, max_seqlen: int | None = None,
                   scale: float | None = None, *, eps: float = 1e-5, out=None, lse=None, stream=None,
                   compute_units: int | None = None, workspace=None):
    """Attention forward with Q's RMSNorm + partial RoPE applied in the kernel's Q-tile load.

    Args:
      q: bfloat16 raw queries ``[total_tokens, heads, 128]``; k (already normalised and
        rotated, e.g. by ``norm_rope``) and v as for ``attn_fwd``.
      q_weight: bfloat16 ``[128]``; cos, sin: bfloat16 ``[total_tokens, R]`` per-token tables,
        or None (R = 0).
      cu_seqlens, max_seqlen, scale, out, lse, stream: as for ``attn_fwd``; eps the RMSNorm epsilon.
      compute_units, workspace: when ``compute_units`` is given, the launch is
        ``lsv_attn_fwd_qnorm_tail`` (the last, partial round of query tiles cut into key ranges),
        with ``workspace`` as for ``attn_fwd_tail``.

    Returns:
      ``(out, lse)``, equal bit for bit to ``attn_fwd(norm_rope(q, q_weight, cos, sin), k, v, ...)``
      (to ``attn_fwd_tail(norm_rope(q, ...), ..., compute_units=...)`` with ``compute_units``).
    """
    import torch
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [total_tokens, heads, head_dim] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q.device
    if dev.type != "cuda" or any(t.device != dev for t in (k, v, cu_seqlens, q_weight)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q.shape
    if q_weight.dtype != torch.bfloat16 or q_weight.shape != (dim,) or not q_weight.is_contiguous():
        raise ValueError("q_weight must be a contiguous bfloat16 [head_dim] tensor")
    rd, cos, sin = _tables(cos, sin, total, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    mine = []
    if out is None:
        out = torch.empty_like(q)
        mine.append(out)
    if lse is None:
        lse = torch.empty((heads, total), dtype=torch.float32, device=dev)
        mine.append(lse)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != dev:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's GPU")
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev:
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor on q's GPU")
    if compute_units is not None:
        need = lsv_attn_fwd_tail_workspace_size(compute_units)
        if need < 0:
            raise ValueError("compute_units must be a positive multiple of 8")
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            mine.append(workspace)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous buffer on the same GPU")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), q_weight.data_ptr(), 0 if cos is None else cos.data_ptr(),
            0 if sin is None else sin.data_ptr(), rd, eps, out.data_ptr(), lse.data_ptr(), cu_seqlens.data_ptr(),
            cu_seqlens.numel() - 1, max_seqlen, total, heads, dim, scale)
    with torch.cuda.device(dev):
        if compute_units is None:
            rc = lsv_attn_fwd_qnorm(*args, s.cuda_stream)
        else:
            rc = lsv_attn_fwd_qnorm_tail(*args, compute_units, workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_qnorm" if compute_units is None else "lsv_attn_fwd_qnorm_tail")
    return out, lse


def _fp8_args(q8, k8, v8, cu_seqlens, max_seqlen, scale, out, lse):
    """Checks the FP8 forward's tensors and fills in the defaults; returns
    (max_seqlen, scale, out, lse, the buffers allocated here)."""
    import torch
    tensors = (q8, k8, v8)
    if any(t.element_size() != 1 or t.is_floating_point() and t.dtype != torch.float8_e4m3fn for t in tensors):
        raise ValueError("q8, k8, v8 must be uint8 or float8_e4m3fn")
    if q8.dim() != 3 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8, v8 must share one [total_tokens, heads, head_dim] shape")
    if not all(t.is_contiguous() for t in tensors):
        raise ValueError("q8, k8, v8 must be contiguous")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    dev = q8.device
    if dev.type != "cuda" or any(t.device != dev for t in (k8, v8, cu_seqlens)):
        raise ValueError("all tensors must be on the same GPU")
    total, heads, dim = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    mine = []
    if out is None:
        out = torch.empty((total, heads, dim), dtype=torch.bfloat16, device=dev)
        mine.append(out)
    if lse is None:
        lse = torch.empty((heads, total), dtype=torch.float32, device=dev)
        mine.append(lse)
    if tuple(out.shape) != (total, heads, dim) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [total_tokens, heads, head_dim] tensor")
    if lse.shape != (heads, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [heads, total_tokens] tensor")
    if out.device != dev or lse.device != dev:
        raise ValueError("out and lse must be on the same GPU as q8")
    return max_seqlen, scale, out, lse, mine


def attn_fwd_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, cu_seqlens,
                 max_seqlen: int | None = None, scale: float | None = None, *, out=None, lse=None, stream=None):
    """FP8 attention forward on torch tensors (one GPU).

    Args:
      q8, k8, v8: ``[total_tokens, n_heads, 128]`` e4m3 bytes (``torch.uint8`` or
        ``torch.float8_e4m3fn``), contiguous.
      descale_q, descale_k, descale_v: per-tensor descales (real value = descale * byte value).
      cu_seqlens, max_seqlen, scale, out, lse, stream: as for ``attn_fwd``.

    Returns:
      ``(out, lse)``: bfloat16 ``[T, H, 128]`` and float32 ``[H, T]``.
    """
    import torch
    max_seqlen, scale, out, lse, mine = _fp8_args(q8, k8, v8, cu_seqlens, max_seqlen, scale, out, lse)
    dev = q8.device
    total, heads, dim = q8.shape
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), descale_q, descale_k, descale_v,
                              out.data_ptr(), lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                              max_seqlen, total, heads, dim, scale, s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_fp8")
    return out, lse


def attn_fwd_fp8_tail(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, cu_seqlens,
                      max_seqlen: int | None = None, scale: float | None = None, *, compute_units: int | None = None,
                      out=None, lse=None, workspace=None, stream=None):
    """FP8 attention forward that cuts the query tiles of the last, partial round of workgroups
    into key ranges (``lsv_attn_fwd_fp8_tail``). Arguments as for ``attn_fwd_fp8``;
    ``compute_units`` and ``workspace`` as for ``attn_fwd_tail``. Returns ``(out, lse)``."""
    import torch
    max_seqlen, scale, out, lse, mine = _fp8_args(q8, k8, v8, cu_seqlens, max_seqlen, scale, out, lse)
    dev = q8.device
    total, heads, dim = q8.shape
    if compute_units is None:
        compute_units = lsv_device_peak(dev.index if dev.index is not None else torch.cuda.current_device())[1]
    need = lsv_attn_fwd_tail_workspace_size(compute_units)
    if need < 0:
        raise ValueError("compute_units must be a positive multiple of 8")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        mine.append(workspace)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same GPU")
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    _keep_for(s, *mine)
    with torch.cuda.device(dev):
        rc = lsv_attn_fwd_fp8_tail(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), descale_q, descale_k, descale_v,
                                   out.data_ptr(), lse.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                   max_seqlen, total, heads, dim, scale, compute_units, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), s.cuda_stream)
    if rc != LSV_OK:
        raise LsvError(rc, "lsv_attn_fwd_fp8_tail")
    return out, lse
