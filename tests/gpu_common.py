"""Shared helpers for the GPU parity tests: moving bf16 bit arrays to and from the device,
comparing kernel outputs with the fp64 oracle at the stated tolerances, the query tiles a tail
plan cuts, and the FP8 tail launch beside the plain one."""

from __future__ import annotations

import sys

import numpy as np

from oracle import attention_fp64, bf16_bits_to_f64

# Tolerances: bf16 output vs the unrounded fp64 oracle, fp32 LSE vs fp64 LSE.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def from_dev(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_kernel(inp, device, *, out_fill=None, lse_fill=None, max_seqlen=None, n_split=1):
    """Run the HIP path on an ``inputs.Inputs`` (``lsv_attn_fwd``, or ``lsv_attn_fwd_split`` with
    ``n_split`` key ranges); returns (out bits [T,H,D], lse [H,T])."""
    import torch
    import long_sequence_video_amd as lsv
    q, k, v = (to_dev(x, device) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    out = torch.empty_like(q)
    lse = torch.empty((inp.n_heads, inp.total_tokens), dtype=torch.float32, device=device)
    if out_fill is not None:
        out.view(torch.int16).fill_(int(np.int16(np.uint16(out_fill))))
    if lse_fill is not None:
        lse.fill_(lse_fill)
    ms = inp.max_seqlen if max_seqlen is None else max_seqlen
    if n_split == 1:
        lsv.attn_fwd(q, k, v, cu, ms, inp.scale, out=out, lse=lse)
    else:
        lsv.attn_fwd_split(q, k, v, cu, ms, inp.scale, n_split, out=out, lse=lse)
    torch.cuda.synchronize(device)
    return from_dev(out), lse.cpu().numpy()


def sample_rows(inp, per_segment: int, seed: int, tile: int = 128) -> np.ndarray:
    """Rows to check: the first and last ``tile`` rows of every segment, plus random rows."""
    rng = np.random.default_rng(seed)
    rows = []
    cu = inp.cu_seqlens.astype(np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        rows.append(np.arange(a, min(b, a + tile)))
        rows.append(np.arange(max(a, b - tile), b))
        rows.append(rng.integers(a, b, size=per_segment))
    return np.unique(np.concatenate(rows)) if rows else np.zeros(0, np.int64)


def compare(inp, out_bits, lse, rows=None, *, label=""):
    """Oracle check of the kernel output on ``rows`` (default: all). Returns the error stats."""
    ref_o, ref_lse, rows = attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale, rows=rows)
    got_o = bf16_bits_to_f64(out_bits[rows])
    got_lse = lse[:, rows].astype(np.float64)
    err = np.abs(got_o - ref_o)
    lerr = np.abs(got_lse - ref_lse)
    stats = dict(o_max=float(err.max(initial=0.0)), o_mean=float(err.mean()) if err.size else 0.0,
                 lse_max=float(lerr.max(initial=0.0)), rows=int(len(rows)))
    say(f"[{label}] {stats}")
    assert np.isfinite(got_o).all(), "non-finite output"
    assert np.isfinite(got_lse).all(), "non-finite LSE"
    assert stats["o_max"] <= O_MAX_ABS, stats
    assert stats["o_mean"] <= O_MEAN_ABS, stats
    assert stats["lse_max"] <= LSE_MAX_ABS, stats
    return stats


def tail_tiles(inp, units):
    """The plan's (split, tail logical tiles): XCD x owns logical tiles [x P, (x + 1) P),
    P = ceil(n / 8) (none from n on), and its last n_tail / 8 are the cut ones."""
    import long_sequence_video_amd as lsv
    split, n_tail = lsv.lsv_attn_fwd_tail_plan(len(inp.cu_seqlens) - 1, inp.max_seqlen, inp.n_heads, units)
    n = (inp.max_seqlen + 255) // 256 * (len(inp.cu_seqlens) - 1) * inp.n_heads
    per_xcd, t = -(-n // 8), n_tail // 8
    return split, [x * per_xcd + per_xcd - t + r for x in range(8) for r in range(t)
                   if x * per_xcd + per_xcd - t + r < n]


def whole_tile_rows(inp, units):
    """(token, head) pairs of the query tiles that the plan leaves whole, as a boolean [T, H]."""
    split, tail = tail_tiles(inp, units)
    tiles = (inp.max_seqlen + 255) // 256
    n_seqs = len(inp.cu_seqlens) - 1
    whole = np.ones((inp.total_tokens, inp.n_heads), bool)
    for logical in tail:
        qt, hs = logical % tiles, logical // tiles
        seg, head = hs % n_seqs, hs // n_seqs
        a, b = int(inp.cu_seqlens[seg]), int(inp.cu_seqlens[seg + 1])
        whole[a + 256 * qt:min(b, a + 256 * qt + 256), head] = False
    return whole, split, len(tail)


def run_fp8_tail(f8, device, units=None, *, out_fill=None):
    """lsv_attn_fwd_fp8_tail and lsv_attn_fwd_fp8 on the same inputs: (out, lse, ref_out, ref_lse)."""
    import torch
    import long_sequence_video_amd as lsv
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(device) for x in (f8.q, f8.k, f8.v))
    cu = torch.from_numpy(f8.cu_seqlens.astype(np.int32)).to(device)
    out = torch.empty(f8.q.shape, dtype=torch.bfloat16, device=device)
    lse = torch.empty((f8.n_heads, f8.total_tokens), dtype=torch.float32, device=device)
    if out_fill is not None:
        out.view(torch.int16).fill_(int(np.int16(np.uint16(out_fill))))
        lse.fill_(-7.0)
    lsv.attn_fwd_fp8_tail(q, k, v, f8.descale_q, f8.descale_k, f8.descale_v, cu, f8.max_seqlen, f8.scale,
                          compute_units=units, out=out, lse=lse)
    ref_o, ref_l = lsv.attn_fwd_fp8(q, k, v, f8.descale_q, f8.descale_k, f8.descale_v, cu, f8.max_seqlen, f8.scale)
    torch.cuda.synchronize(device)
    return from_dev(out), lse.cpu().numpy(), from_dev(ref_o), ref_l.cpu().numpy()
