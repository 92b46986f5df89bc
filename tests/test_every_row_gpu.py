"""Every query row of the large workloads against the fp64 oracles: the whole output, where the
other full-size tests check the first and last tiles of each segment, the cut tiles and random rows.

The forward launches are the ones the benchmark times (``lsv_attn_fwd_tail``,
``lsv_attn_fwd_fp8_tail`` on the device's compute units). The BF16 forward at 38,000 x 56 with
RMS-normalised Q and K (4.1e13 fp64 flops for the oracle, about a minute on 16 host cores) runs by
default. The others take minutes of host time each and run when the environment asks for them:
``LSV_EVERY_ROW_PACK=1`` the BF16 forward on the 161,394-token pack (3.6e14 flops, about 8
minutes), ``LSV_EVERY_ROW_FP8=1`` the FP8 forward on the same pack, ``LSV_EVERY_ROW_BWD=1`` dQ, dK
and dV at 38,000 x 56. Each prints one line per head group as it goes.

Bars: those of the sampled checks. BF16 forward: O within 2e-2 (max-abs) and 2e-3 (mean-abs over
every element) of the unrounded fp64 oracle, LSE within 1e-3. FP8 forward and backward: the bars
their own parity tests derive (``tests/test_fp8_gpu.py``, ``tests/test_bwd_gpu.py``)."""

from __future__ import annotations

import os
import time

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import attention_fp64, bf16_bits_to_f64
from tests.gpu_common import LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

HEAD_GROUP = 16  # the oracle's parallelism is one (segment, head) pair per thread


def run_bench_launch(inp, device):
    """The benchmark's launch of the forward; returns (O bits [T, H, D], LSE [H, T]) on the host."""
    import torch
    import long_sequence_video_amd as lsv
    units = lsv.lsv_device_peak(0)[1]
    q, k, v = (to_dev(x, device) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    out = torch.empty_like(q)
    out.view(torch.int16).fill_(0x7FC0)  # NaN: a row the kernel skips cannot pass
    lse = torch.full((inp.n_heads, inp.total_tokens), float("nan"), dtype=torch.float32, device=device)
    ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(units), dtype=torch.uint8, device=device)
    lsv.attn_fwd_tail(q, k, v, cu, inp.max_seqlen, inp.scale, compute_units=units, out=out, lse=lse,
                      workspace=ws)
    torch.cuda.synchronize(device)
    o_bits, lse_h = from_dev(out), lse.cpu().numpy()
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return o_bits, lse_h


def bf16_oracle(inp):
    return lambda q, k, v, rows: attention_fp64(q, k, v, inp.cu_seqlens, inp.scale, rows=rows)


def check_every_row(inp, o_bits, lse, label, oracle=None, bars=(O_MAX_ABS, O_MEAN_ABS, LSE_MAX_ABS),
                    row_chunk=None):
    """``oracle(q, k, v, rows)`` (default: the BF16 one) over every row, one segment and head
    group per call (and at most ``row_chunk`` rows per call, for an oracle that forms a
    (segment, head)'s scores for all requested rows at once), on the head-sliced inputs; returns
    the error stats over all of them."""
    oracle = oracle or bf16_oracle(inp)
    cu = inp.cu_seqlens.astype(np.int64)
    o_max = lse_max = o_sum = 0.0
    count = 0
    t0 = time.perf_counter()
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        step = row_chunk or (b - a)
        for h0 in range(0, inp.n_heads, HEAD_GROUP):
            h1 = min(inp.n_heads, h0 + HEAD_GROUP)
            part = [np.ascontiguousarray(x[:, h0:h1, :]) for x in (inp.q, inp.k, inp.v)]
            for r0 in range(a, b, step):
                r1 = min(b, r0 + step)
                ref_o, ref_lse, _ = oracle(*part, np.arange(r0, r1, dtype=np.int64))
                got_o = bf16_bits_to_f64(o_bits[r0:r1, h0:h1, :])
                got_lse = lse[h0:h1, r0:r1].astype(np.float64)
                assert np.isfinite(got_o).all() and np.isfinite(got_lse).all(), (label, r0, r1, h0)
                err = np.abs(got_o - ref_o)
                o_max = max(o_max, float(err.max()))
                o_sum += float(err.sum())
                count += err.size
                lse_max = max(lse_max, float(np.abs(got_lse - ref_lse).max()))
                del ref_o, ref_lse, got_o, err
            say(f"[{label}] segment [{a}, {b}) heads {h0}..{h1 - 1}: O max {o_max:.3e}, "
                f"LSE max {lse_max:.3e} so far ({time.perf_counter() - t0:.0f} s)")
            del part
    stats = dict(rows=int(sum(b - a for a, b in zip(cu[:-1], cu[1:]))), o_max=o_max, o_mean=o_sum / count,
                 lse_max=lse_max, oracle_s=round(time.perf_counter() - t0, 1))
    say(f"[{label}] every row: {stats}")
    o_bar, mean_bar, lse_bar = bars
    assert stats["o_max"] <= o_bar and stats["o_mean"] <= mean_bar and stats["lse_max"] <= lse_bar, stats
    return stats


def test_every_row_at_38000_h56(gpu):
    inp = gen.make_config("h3_s38000_h56")
    say("case every row h3_s38000_h56")
    o_bits, lse = run_bench_launch(inp, gpu)
    check_every_row(inp, o_bits, lse, "h3_s38000_h56")


@pytest.mark.skipif(os.environ.get("LSV_EVERY_ROW_PACK") != "1",
                    reason="about 8 minutes of host time; set LSV_EVERY_ROW_PACK=1")
def test_every_row_of_the_pack(gpu):
    inp = gen.make_config("varlen_19394_38000_104000_h56")
    say("case every row varlen_19394_38000_104000_h56")
    o_bits, lse = run_bench_launch(inp, gpu)
    check_every_row(inp, o_bits, lse, "varlen_19394_38000_104000_h56")


@pytest.mark.skipif(os.environ.get("LSV_EVERY_ROW_FP8") != "1",
                    reason="about 8 minutes of host time; set LSV_EVERY_ROW_FP8=1")
def test_every_row_fp8_pack(gpu):
    import torch
    import long_sequence_video_amd as lsv
    from oracle import attention_fp8_fp64
    from tests.test_fp8_gpu import LSE_MAX, O_MAX, O_MEAN
    f8 = gen.quantize_fp8(gen.make_config("varlen_19394_38000_104000_h56"))
    say("case every row fp8 varlen_19394_38000_104000_h56")
    units = lsv.lsv_device_peak(0)[1]
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(gpu) for x in (f8.q, f8.k, f8.v))
    cu = torch.from_numpy(f8.cu_seqlens.astype(np.int32)).to(gpu)
    out = torch.empty(f8.q.shape, dtype=torch.bfloat16, device=gpu)
    out.view(torch.int16).fill_(0x7FC0)
    lse = torch.full((f8.n_heads, f8.total_tokens), float("nan"), dtype=torch.float32, device=gpu)
    ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(units), dtype=torch.uint8, device=gpu)
    lsv.attn_fwd_fp8_tail(q, k, v, f8.descale_q, f8.descale_k, f8.descale_v, cu, f8.max_seqlen, f8.scale,
                          compute_units=units, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize(gpu)
    o_bits, lse_h = from_dev(out), lse.cpu().numpy()
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()

    def oracle(q8, k8, v8, rows):
        return attention_fp8_fp64(q8, k8, v8, f8.descale_q, f8.descale_k, f8.descale_v, f8.cu_seqlens, f8.scale,
                                  rows=rows)
    # 1,024 rows x 104,000 keys x (scores + weights) x 16 threads: about 27 GB of fp64 at once
    check_every_row(f8, o_bits, lse_h, "fp8 varlen_19394_38000_104000_h56", oracle, (O_MAX, O_MEAN, LSE_MAX),
                    row_chunk=1024)


@pytest.mark.skipif(os.environ.get("LSV_EVERY_ROW_BWD") != "1",
                    reason="about 5 minutes of host time; set LSV_EVERY_ROW_BWD=1")
def test_every_row_bwd_at_38000_h56(gpu):
    """dQ, dK and dV of every row and head at 38,000 x 56 (RMS-normalised Q and K), one launch.
    As in the sampled backward checks, the kernel's O and LSE inputs are the oracle's fp64 forward
    rounded to bf16 and fp32; the bar is the backward's relative one, per gradient tensor and head
    group of 8."""
    import torch
    import long_sequence_video_amd as lsv
    from oracle import attention_bwd_fp64
    from tests.test_bwd_gpu import _dout, compare, run_bwd
    inp = gen.make_config("h3_s38000_h56")
    do = _dout(inp, 1004)
    say("case every row bwd h3_s38000_h56")
    q, k, v = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(gpu)
    out, lse = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale)
    torch.cuda.synchronize(gpu)
    out_bits, lse_h = from_dev(out), lse.cpu().numpy()
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    refs = []
    t0 = time.perf_counter()
    for h0 in range(0, inp.n_heads, 8):
        hs = list(range(h0, min(inp.n_heads, h0 + 8)))
        sub = lambda x: np.ascontiguousarray(x[:, hs])  # noqa: E731
        ref = attention_bwd_fp64(sub(inp.q), sub(inp.k), sub(inp.v), sub(do), inp.cu_seqlens, inp.scale,
                                 return_forward=True)
        for i, h in enumerate(hs):
            out_bits[:, h] = gen.f64_to_bf16_bits(ref["o"][:, i])
            lse_h[h] = ref["lse"][i].astype(np.float32)
        del ref["o"], ref["lse"]
        refs.append((hs, ref))
        say(f"[bwd every row] oracle heads {hs[0]}..{hs[-1]} ({time.perf_counter() - t0:.0f} s)")
    grads = run_bwd(inp, do, gpu, out_bits=out_bits, lse=lse_h)
    for hs, ref in refs:
        compare(inp, do, grads, label=f"bwd every row heads {hs[0]}..{hs[-1]}", ref=ref, heads=hs)
