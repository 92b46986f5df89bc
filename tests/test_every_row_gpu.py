"""Every query row of the large forward workloads against the fp64 oracle: the whole output,
where the other full-size tests check the first and last tiles of each segment, the cut tiles and
random rows.

The launch is the one the benchmark times (``lsv_attn_fwd_tail`` on the device's compute units).
38,000 x 56 with RMS-normalised Q and K (4.1e13 fp64 flops for the oracle, about a minute on 16
host cores) runs by default. The 161,394-token pack (3.6e14 flops, about 8 minutes) runs only when
the environment sets ``LSV_EVERY_ROW_PACK=1``; it prints one line per head group as it goes.

Bars: bf16 O within 2e-2 (max-abs) and 2e-3 (mean-abs over every element) of the unrounded fp64
oracle, fp32 LSE within 1e-3, as for the sampled checks."""

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


def check_every_row(inp, o_bits, lse, label):
    """Oracle over every row, one segment and head group per call; the error stats over all."""
    cu = inp.cu_seqlens.astype(np.int64)
    o_max = lse_max = o_sum = 0.0
    count = 0
    t0 = time.perf_counter()
    for a, b in zip(cu[:-1], cu[1:]):
        if b <= a:
            continue
        rows = np.arange(a, b, dtype=np.int64)
        for h0 in range(0, inp.n_heads, HEAD_GROUP):
            h1 = min(inp.n_heads, h0 + HEAD_GROUP)
            part = [np.ascontiguousarray(x[:, h0:h1, :]) for x in (inp.q, inp.k, inp.v)]
            ref_o, ref_lse, _ = attention_fp64(*part, inp.cu_seqlens, inp.scale, rows=rows)
            got_o = bf16_bits_to_f64(o_bits[a:b, h0:h1, :])
            got_lse = lse[h0:h1, a:b].astype(np.float64)
            assert np.isfinite(got_o).all() and np.isfinite(got_lse).all(), (label, a, b, h0)
            err = np.abs(got_o - ref_o)
            o_max = max(o_max, float(err.max()))
            o_sum += float(err.sum())
            count += err.size
            lse_max = max(lse_max, float(np.abs(got_lse - ref_lse).max()))
            say(f"[{label}] segment [{a}, {b}) heads {h0}..{h1 - 1}: O max {o_max:.3e}, "
                f"LSE max {lse_max:.3e} so far ({time.perf_counter() - t0:.0f} s)")
            del ref_o, ref_lse, got_o, err, part
    stats = dict(rows=int(sum(b - a for a, b in zip(cu[:-1], cu[1:]))), o_max=o_max, o_mean=o_sum / count,
                 lse_max=lse_max, oracle_s=round(time.perf_counter() - t0, 1))
    say(f"[{label}] every row: {stats}")
    assert stats["o_max"] <= O_MAX_ABS and stats["o_mean"] <= O_MEAN_ABS and stats["lse_max"] <= LSE_MAX_ABS
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
