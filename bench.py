"""Benchmark: BF16 attention forward TFLOP/s on MI355X (flops counted as sum 4 * S^2 * H * D).

One step = one attention forward over the whole packed workload (one kernel launch),
inputs already resident in HBM. Default workload: the varlen pack of three MiniMax-H3
clips, 19,394 + 38,000 + 104,000 tokens x 56 heads x 128 (161,394 tokens; 3.623e14 flops
per step). Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                  [--no-prologue] [--prologue-only] [--no-bwd] [--bwd-only] [--no-fp8] [--fp8-only]
                  [--no-gemm-ref] [--gemm-ref-only]
  python bench.py --copy-bytes N   # a plain device copy of N bytes, to calibrate HBM counters

An object ``attn_fwd_fp8`` times the FP8 (e4m3) forward on the same pack quantised per tensor,
with the same flop count, against MI355X's dense FP8 peak (5.0 PFLOP/s); with the default
``--split auto`` it runs lsv_attn_fwd_fp8_tail, the launch that cuts the last, partial round of
query tiles into key ranges when the plan cuts any. Its ``legs`` time the same on the sp=4 share
(19,394 x 14), whose last round is one-sixth full.

An object ``attn_bwd`` times the backward (dQ, dK, dV; deterministic, two kernels) on the
same pack, counted the usual way as 2.5 x the forward's flops (the five products of the
textbook backward); its roofline.frac is stated on that count. The kernels execute seven
products (the dQ pass recomputes S and dP instead of accumulating dQ with atomics), reported
apart as ``mfma_flops_executed`` / ``frac_executed``. O and LSE come from the forward kernel.
Not part of ``value``.

An object ``forward_legs`` times the same forward on each of the other workloads (the
104,000-token segment of the pack alone, the 40% target row; 4,096 x 56 with boosted keys;
the sp=4 shares 19,394 x 14 and 38,000 x 14; 38,000 x 56; the tiny 256 x 4 case), each with its own steps and
the same automatic key split as the headline. Not part of ``value``. One more leg,
``fallback_s38000_h56``, is 38,000 x 56 with every query's first key tile scoring far below the
rest, so that every workgroup's fixed-reference pass overflows and reruns on the exact path;
its ``vs_fast_path`` is its time over the plain 38,000 x 56 leg's.

A second object, ``qkv_prologue``, times the fused QKV prologue (QK RMSNorm + partial RoPE +
V copy, the pass that feeds attention) on the same token count: 161,394 tokens x 56 heads x
128, rotary width 96. It is bound by HBM and reported in GB/s against 8 TB/s; it is not
part of ``value``. ``qkv_prologue_fused_q`` times prologue + forward on the pack two ways:
the stacked prologue then the forward, and the K-only prologue then the forward that
normalises and rotates Q in its Q-tile load (six planes of prologue traffic against two).

An object ``mfma_reference`` times a plain library GEMM (torch.matmul, i.e. hipBLASLt, bf16,
16384^3, 50 calls back to back) on the same GPU: the dense matrix throughput a tuned library
sustains on this chip at its power limit, the practical ceiling the attention kernels are compared with
(``vs_library_gemm``). ``attn_fwd_fp8`` carries the same for e4m3 (torch._scaled_mm). They are
calibrations, not part of ``value``.

roofline.traffic (HBM bytes per launch) comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE
summary committed under profiles/ for this workload, scaled by the same counters on a copy of
known size; it is null when that summary was taken on a different kernel source or device header.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense BF16 MFMA peak (2.5 PFLOP/s)
DEFAULT_CONFIG = "varlen_19394_38000_104000_h56"
# The segment of the default pack that the 40% target is stated for, run alone.
EXTRA_CONFIGS = {"h56_s104000": dict(seqlens=[104000], heads=56, seed=1005),
                 # one sp=4 rank's 14-head share of the 38,000-token clip (RMS-normalised Q/K)
                 "sp4_share_s38000_h14": dict(seqlens=[38000], heads=14, seed=1008, rms_qk=True),
                 # 38,000 x 56 with every query's first key tile ~113 nats below the rest: every
                 # workgroup's fixed-reference pass overflows and reruns on the exact path.
                 "fallback_s38000_h56": dict(seqlens=[38000], heads=56, seed=1004, rms_qk=True,
                                             low_first_tile=80.0)}


KERNEL_SOURCE = os.path.join(ROOT, "long_sequence_video_amd", "csrc", "attn_fwd.hip")
PROLOGUE_SOURCE = os.path.join(ROOT, "long_sequence_video_amd", "csrc", "qkv_prologue.hip")
FP8_SOURCE = os.path.join(ROOT, "long_sequence_video_amd", "csrc", "attn_fwd_fp8.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "{kernel}_{workload}_hbm_traffic.md")


def kernel_source_sha256(path: str = KERNEL_SOURCE) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def kernel_device_headers(path: str = KERNEL_SOURCE) -> list:
    """The device-code headers a kernel source includes from its own folder (tile_ops.h: the
    MFMA, LDS and copy helpers). lsv.h, in include/, declares the C ABI only."""
    here = os.path.dirname(path)
    found = []
    for line in open(path):
        m = re.match(r'\s*#include\s+"([^"]+)"', line)
        if m and os.path.exists(os.path.join(here, m.group(1))):
            found.append(os.path.join(here, m.group(1)))
    return found


def kernel_headers_sha256(path: str = KERNEL_SOURCE) -> str:
    """SHA-256 over the device headers of ``path``, in include order."""
    h = hashlib.sha256()
    for header in kernel_device_headers(path):
        h.update(open(header, "rb").read())
    return h.hexdigest()


def profile_fields(workload: str, kernel_source: str = KERNEL_SOURCE, kernel: str = "attn_fwd"):
    """(machine-readable fields, summary path) of the committed counter summary for this
    workload, if it was taken on the current kernel source; else (None, reason)."""
    path = TRAFFIC_SUMMARY.format(kernel=kernel, workload=workload)
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            key, val = line[2:].split(":", 1)
            quoted = re.search(r"`([^`]*)`", val)
            fields[key.strip()] = quoted.group(1) if quoted else val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256(kernel_source):
        return None, "counter summary predates the current kernel source"
    if kernel_device_headers(kernel_source) and \
            fields.get("kernel_headers_sha256") != kernel_headers_sha256(kernel_source):
        return None, "counter summary predates the current device headers"
    return fields, os.path.relpath(path, ROOT)


def measured_traffic(workload: str, kernel_source: str = KERNEL_SOURCE, kernel: str = "attn_fwd"):
    """(HBM bytes per launch, summary path) from the committed counter summary, if it was taken
    on the current kernel source; else (None, reason)."""
    fields, src = profile_fields(workload, kernel_source, kernel)
    if fields is None:
        return None, src
    try:
        return float(fields["hbm_bytes_per_launch"]), src
    except (KeyError, ValueError):
        return None, "counter summary lacks hbm_bytes_per_launch"


def measured_mfma_flops(workload: str, kernel_source: str, kernel: str):
    """Matrix flops one launch executes (the SQ_INSTS_VALU_MFMA_MOPS_* counter x 512) from the
    committed counter summary, if taken on the current kernel source; else None."""
    fields, _ = profile_fields(workload, kernel_source, kernel)
    try:
        return float(fields["mfma_flops_executed_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int, steps: int):
    """A plain device-to-device copy of nbytes, repeated: the reference kernel for the HBM
    counters (it reads and writes exactly nbytes per launch)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes": nbytes, "launches": steps}), flush=True)


PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth (8 TB/s)
PROLOGUE_CONFIG = "prologue_s161394_h56"


def bench_prologue(steps: int, warmup: int):
    """Time the fused QKV prologue on its bench workload; returns the JSON object."""
    import torch
    import long_sequence_video_amd as lsv
    from long_sequence_video_amd import inputs as gen
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = gen.make_prologue_config(PROLOGUE_CONFIG)
    log(f"generated {PROLOGUE_CONFIG} in {time.perf_counter() - t0:.1f} s")
    to = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    q, k, v, qw, kw, cos, sin = (to(x) for x in (inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin))
    b, s, h, d = inp.shape
    out = torch.empty((3 * b, s, h, d), dtype=torch.bfloat16, device=dev)

    def step():
        lsv.qkv_prologue(q, k, v, qw, kw, cos, sin, eps=inp.eps, out=out)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    nbytes = inp.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"{PROLOGUE_CONFIG}: {ms:.3f} ms, {gbs:.0f} GB/s, {100 * gbs / PEAK_HBM_GBS:.1f}% of HBM peak")
    traffic, traffic_src = measured_traffic(PROLOGUE_CONFIG, kernel_source=PROLOGUE_SOURCE, kernel="qkv_prologue")
    del q, k, v, qw, kw, cos, sin, out
    torch.cuda.empty_cache()
    return {
        "workload": PROLOGUE_CONFIG, "shape": [b, s, h, d], "rotary_dim": inp.rotary_dim,
        "ms_per_call": round(ms, 4), "steps": steps,
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_unit": "HBM bytes per launch",
            "traffic_source": traffic_src, "algorithmic_hbm_bytes": nbytes, "kernel": "qkv_prologue_kernel",
        },
    }


def bench_qnorm(steps: int, warmup: int):
    """The forward with the QKV prologue in front of it on the 161,394-token pack x 56 heads
    (R = 96, each segment's own RoPE positions), two ways: the stacked prologue (Q, K, V planes)
    then the forward, and lsv_norm_rope on K then the forward with Q's norm and rotation in its
    Q-tile load. Both forwards are the headline's launch (the tail split on the device's compute
    units: lsv_attn_fwd_tail and lsv_attn_fwd_qnorm_tail). Returns the JSON object (per-part
    times, and the prologue bytes each way)."""
    import torch
    import long_sequence_video_amd as lsv
    from long_sequence_video_amd import inputs as gen
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = gen.generate_qnorm([19394, 38000, 104000], 56, 96, seed=1008, name="qnorm_varlen_161394_h56")
    log(f"generated {inp.name} in {time.perf_counter() - t0:.1f} s")
    to = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    q, k, v, qw, kw, cos, sin = (to(x) for x in (inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin))
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    t, h = inp.total_tokens, inp.n_heads
    stacked = torch.empty((3, t, h, 128), dtype=torch.bfloat16, device=dev)
    kn = torch.empty_like(k)
    out = torch.empty_like(q)
    lse = torch.empty((h, t), dtype=torch.float32, device=dev)
    ms = inp.max_seqlen
    _, n_cus, _ = lsv.lsv_device_peak(0)
    ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(n_cus), dtype=torch.uint8, device=dev)
    parts = {
        "two_pass": [lambda: lsv.qkv_prologue(q, k, v, qw, kw, cos, sin, eps=inp.eps, out=stacked),
                     lambda: lsv.attn_fwd_tail(stacked[0], stacked[1], stacked[2], cu, ms, inp.scale,
                                               compute_units=n_cus, out=out, lse=lse, workspace=ws)],
        "fused_q": [lambda: lsv.norm_rope(k, kw, cos, sin, eps=inp.eps, out=kn),
                    lambda: lsv.attn_fwd_qnorm(q, kn, v, qw, cos, sin, cu, ms, inp.scale, eps=inp.eps, out=out,
                                               lse=lse, compute_units=n_cus, workspace=ws)],
    }
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, (pro, att) in parts.items():
        for _ in range(warmup):
            pro()
            att()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
        torch.cuda.synchronize(dev)
        ev[0].record(stream)
        for i in range(steps):
            pro()
            ev[2 * i + 1].record(stream)
            att()
            ev[2 * i + 2].record(stream)
        torch.cuda.synchronize(dev)
        pro_ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
        att_ms = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps)) / steps
        res[name] = {"prologue_ms": round(pro_ms, 4), "attention_ms": round(att_ms, 4),
                     "total_ms": round(pro_ms + att_ms, 4)}
        log(f"{inp.name} {name}: prologue {pro_ms:.3f} ms + attention {att_ms:.3f} ms")
    plane = t * h * 128 * 2
    res.update({"workload": inp.name, "rotary_dim": 96, "steps": steps,
                "prologue_hbm_bytes": {"two_pass": 6 * plane, "fused_q": 2 * plane},
                "attention_tflops_fused_q": round(inp.flops() / (res["fused_q"]["attention_ms"] * 1e-3) / 1e12, 2)})
    del q, k, v, qw, kw, cos, sin, stacked, kn, out, lse, ws
    torch.cuda.empty_cache()
    return res


PEAK_FP8_TFLOPS = 5000.0  # MI355X published dense FP8 MFMA peak (5.0 PFLOP/s)
FP8_LEG = "sp4_share_s19394_h14"  # the FP8 forward's second workload in the default run


def bench_fp8(name: str, steps: int, warmup: int, split="auto"):
    """Time the FP8 forward on workload ``name`` quantised per tensor; returns the JSON object.
    With ``split`` "auto" the launch is lsv_attn_fwd_fp8_tail (the last, partial round of query
    tiles cut into key ranges when the plan cuts any, else lsv_attn_fwd_fp8); otherwise
    lsv_attn_fwd_fp8."""
    import torch
    import long_sequence_video_amd as lsv
    from long_sequence_video_amd import inputs as gen
    dev = torch.device("cuda:0")
    f8 = gen.quantize_fp8(make_inputs(name))
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (f8.q, f8.k, f8.v))
    cu = torch.from_numpy(f8.cu_seqlens).to(dev)
    out = torch.empty(f8.q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((f8.n_heads, f8.total_tokens), dtype=torch.float32, device=dev)
    _, n_cus, _ = lsv.lsv_device_peak(0)
    ranges, tail_tiles = lsv.lsv_attn_fwd_tail_plan(len(f8.cu_seqlens) - 1, f8.max_seqlen, f8.n_heads, n_cus)
    tail = split == "auto" and ranges > 1
    ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(n_cus), dtype=torch.uint8, device=dev) if tail else None

    def step():
        if tail:
            lsv.attn_fwd_fp8_tail(q, k, v, f8.descale_q, f8.descale_k, f8.descale_v, cu, f8.max_seqlen, f8.scale,
                                  compute_units=n_cus, out=out, lse=lse, workspace=ws)
        else:
            lsv.attn_fwd_fp8(q, k, v, f8.descale_q, f8.descale_k, f8.descale_v, cu, f8.max_seqlen, f8.scale,
                             out=out, lse=lse)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    tf = f8.flops() / (ms * 1e-3) / 1e12
    log(f"{name} fp8{' (tail split)' if tail else ''}: {ms:.3f} ms, {tf:.1f} TFLOP/s, "
        f"{100 * tf / PEAK_FP8_TFLOPS:.1f}% of the FP8 peak")
    kernel = "attn_fwd_fp8_tail" if tail else "attn_fwd_fp8"
    traffic, traffic_src = measured_traffic(name, kernel_source=FP8_SOURCE, kernel=kernel)
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return {
        "workload": name + " (e4m3, per-tensor descales)", "ms_per_step": round(ms, 4), "steps": steps,
        "key_split": {"tail_ranges": ranges, "tail_tiles": tail_tiles} if tail else 1,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": kernel + "_kernel",
                     # SQ_INSTS_VALU_MFMA_MOPS_F8 x 512: the counted flops, the padding of the
                     # last key tiles and the weight-sum MFMA
                     "mfma_flops_executed": measured_mfma_flops(name, FP8_SOURCE, kernel)},
    }


def bench_backward(name: str, steps: int, warmup: int):
    """Time the attention backward on workload ``name``; returns the JSON object."""
    import torch
    import long_sequence_video_amd as lsv
    from long_sequence_video_amd import inputs as gen
    dev = torch.device("cuda:0")
    inp = make_inputs(name)
    do_bits = gen.normal_bf16(inp.q.size, 7, 9).reshape(inp.q.shape)
    to = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    q, k, v, do = to(inp.q), to(inp.k), to(inp.v), to(do_bits)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    out, lse = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(lsv.lsv_attn_bwd_workspace_size(inp.total_tokens, inp.n_heads), dtype=torch.uint8, device=dev)

    def step():
        lsv.attn_bwd(q, k, v, out, do, lse, cu, inp.max_seqlen, inp.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    fwd = inp.flops()
    counted = 2.5 * fwd
    executed = 3.5 * fwd
    tf = counted / (ms * 1e-3) / 1e12
    tf_exec = executed / (ms * 1e-3) / 1e12
    log(f"{name} backward: {ms:.3f} ms, {tf:.1f} TFLOP/s counted (2.5 x fwd), {100 * tf / PEAK_BF16_TFLOPS:.1f}% "
        f"of peak; {tf_exec:.1f} executed")
    del q, k, v, do, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {
        "workload": name, "ms_per_step": round(ms, 4), "steps": steps,
        "tflops_counted": round(tf, 2), "flops_counted": counted, "counting": "2.5 x sum 4*S^2*H*D",
        # The method's own work is the five products counted above; the roofline is stated on
        # that count. The kernels also recompute S and dP in the dQ pass (seven products):
        "mfma_flops_executed": executed, "tflops_executed": round(tf_exec, 2),
        "frac_executed": round(tf_exec / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": "counted (2.5 x sum 4*S^2*H*D)",
                     "kernels": ["bwd_prep_kernel", "attn_bwd_kernel (dK/dV and dQ passes)"]},
    }


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(name):
    from long_sequence_video_amd import inputs as gen
    if name in gen.CONFIGS:
        return gen.make_config(name)
    if name in EXTRA_CONFIGS:
        return gen.generate(name=name, **EXTRA_CONFIGS[name])
    raise SystemExit(f"unknown config {name!r}; known: {sorted(gen.CONFIGS) + sorted(EXTRA_CONFIGS)}")


def time_forward(inp, steps: int, warmup: int, split="auto"):
    """Time the forward on ``inp`` (resident in HBM): ``steps`` launches after ``warmup``, with
    HIP events on the stream the kernels run on (torch's current stream). Returns (ms per
    launch over the whole timed region, the sorted per-launch times, the key split used)."""
    import torch
    import long_sequence_video_amd as lsv
    dev = torch.device("cuda:0")
    to = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    q, k, v = to(inp.q), to(inp.k), to(inp.v)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((inp.n_heads, inp.total_tokens), dtype=torch.float32, device=dev)
    ms = inp.max_seqlen
    _, n_cus, _ = lsv.lsv_device_peak(0)
    ws = None
    if split == "auto":
        ranges, tail_tiles = lsv.lsv_attn_fwd_tail_plan(len(inp.cu_seqlens) - 1, ms, inp.n_heads, n_cus)
        n_split = {"tail_ranges": ranges, "tail_tiles": tail_tiles} if ranges > 1 else 1
    else:
        n_split = int(split)
    if isinstance(n_split, dict):
        ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(n_cus), dtype=torch.uint8, device=dev)
        log(f"{inp.name}: forward with the last round's {n_split['tail_tiles']} query tiles cut into "
            f"{n_split['tail_ranges']} key ranges (lsv_attn_fwd_tail)")
    elif n_split > 1:
        ws = torch.empty(lsv.lsv_attn_fwd_split_workspace_size(inp.total_tokens, inp.n_heads, n_split),
                         dtype=torch.uint8, device=dev)
        log(f"{inp.name}: forward with {n_split} key ranges per segment (lsv_attn_fwd_split)")

    def step():
        if isinstance(n_split, dict):
            lsv.attn_fwd_tail(q, k, v, cu, ms, inp.scale, compute_units=n_cus, out=out, lse=lse, workspace=ws)
        elif n_split == 1:
            lsv.attn_fwd(q, k, v, cu, ms, inp.scale, out=out, lse=lse)
        else:
            lsv.attn_fwd_split(q, k, v, cu, ms, inp.scale, n_split, out=out, lse=lse, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    # One event between consecutive launches: the first and last bracket the timed steps, and
    # the ones in between give the per-launch distribution (p50 / p95).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize(dev)
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    ms_per_step = marks[0].elapsed_time(marks[-1]) / steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return ms_per_step, per_step, n_split


# The forward legs of the default run: (workload, timed launches) -- about half a second of
# GPU time each, plus a few warmup launches.
FORWARD_LEGS = {"h56_s104000": 4, "s4096_h56_kboost": 400, "sp4_share_s19394_h14": 100, "sp4_share_s38000_h14": 50,
                "h3_s38000_h56": 20,
                "tiny_s256_h4": 400, "fallback_s38000_h56": 8}


def bench_forward_leg(name: str, split="auto"):
    """The forward on one more workload; returns the JSON object."""
    t0 = time.perf_counter()
    inp = make_inputs(name)
    gen_s = time.perf_counter() - t0
    steps = FORWARD_LEGS.get(name, 10)
    ms, per_step, n_split = time_forward(inp, steps, 3 if steps < 50 else 20, split)
    tf = inp.flops() / (ms * 1e-3) / 1e12
    log(f"{name}: {ms:.4f} ms/step, {tf:.1f} TFLOP/s, {100 * tf / PEAK_BF16_TFLOPS:.1f}% of peak "
        f"(generated in {gen_s:.1f} s)")
    return {"workload": name, "seqlens": inp.seqlens, "heads": inp.n_heads, "flops_per_step": inp.flops(),
            "steps": steps, "ms_per_step": round(ms, 5), "p50_ms": round(float(np.percentile(per_step, 50)), 5),
            "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4), "key_split": n_split}


def cpu_baseline(inp, target_seconds: float = 15.0):
    """Time the fp64 oracle on a bounded row sample of the same workload, on this host's cores."""
    from oracle import attention_fp64
    cores = len(os.sched_getaffinity(0))
    cu = inp.cu_seqlens.astype(np.int64)
    segs = [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]
    rng = np.random.default_rng(0)

    def sample(per_seg):
        rows = [np.sort(rng.choice(np.arange(a, b), size=min(per_seg, b - a), replace=False)) for a, b in segs]
        return np.concatenate(rows)

    def flops_of(rows):
        f = 0.0
        for a, b in segs:
            n = int(((rows >= a) & (rows < b)).sum())
            f += 4.0 * n * (b - a) * inp.n_heads * inp.head_dim
        return f

    # calibrate on a sample of ~1 s, then size the timed sample to ~target_seconds
    per_seg = 16
    while True:
        rows = sample(per_seg)
        t0 = time.perf_counter()
        attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale, rows=rows, workers=cores)
        dt = time.perf_counter() - t0
        if dt > 1.0 or per_seg >= 4096:
            break
        per_seg *= 4
    rate = flops_of(rows) / dt
    per_seg = max(1, min(8192, int(per_seg * target_seconds * rate / max(flops_of(rows), 1.0))))
    rows = sample(per_seg)
    t0 = time.perf_counter()
    attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale, rows=rows, workers=cores)
    dt = time.perf_counter() - t0
    f = flops_of(rows)
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{len(rows)} query rows ({per_seg} per segment, all {inp.n_heads} heads) of the same "
                   f"workload against every key of their segment; fp64 numpy oracle, {cores} threads; "
                   f"{f:.3e} flops in {dt:.1f} s"),
        "cpu_model": host_cpu_model(),
        "blas": host_blas(),
    }


def host_cpu_model() -> str | None:
    """The host CPU's model name (/proc/cpuinfo), or None where that file has none."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_blas() -> str | None:
    """numpy's BLAS backend and version. The oracle runs it single-threaded inside each of its
    worker threads, so the thread count is the `cores` figure."""
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        return None
    libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    if not libs:
        return None
    return ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)


def bench_gemm_reference(dtype: str = "bf16", steps: int = 50, warmup: int = 5, n: int = 16384):
    """Time a library GEMM on n x n x n: torch.matmul (hipBLASLt) for ``bf16``, torch._scaled_mm
    (hipBLASLt, e4m3 inputs, unit scales, bf16 output) for ``fp8``; returns the JSON object. The
    default calls run about as long as one attention step, so both meet the same power limit."""
    import torch
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    if dtype == "bf16":
        def call():
            torch.matmul(a, b, out=c)
        name, peak = f"torch.matmul (hipBLASLt), bf16, {n} x {n} x {n}", PEAK_BF16_TFLOPS
    elif dtype == "fp8":
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        b8t = b8.t()  # the column-major second operand _scaled_mm takes
        one = torch.ones((), device=dev, dtype=torch.float32)

        def call():
            torch._scaled_mm(a8, b8t, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        name, peak = f"torch._scaled_mm (hipBLASLt), e4m3 in, bf16 out, {n} x {n} x {n}", PEAK_FP8_TFLOPS
    else:
        raise ValueError(dtype)
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    log(f"library GEMM reference: {dtype} {n}^3 in {ms:.3f} ms, {tf:.1f} TFLOP/s, {100 * tf / peak:.1f}% of peak")
    del a, b, c
    torch.cuda.empty_cache()
    return {"kernel": name, "ms": round(ms, 4), "tflops": round(tf, 2), "frac_of_peak": round(tf / peak, 4),
            "steps": steps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0, help="run the counter-calibration copy instead")
    ap.add_argument("--no-prologue", action="store_true", help="skip the QKV-prologue leg")
    ap.add_argument("--prologue-only", action="store_true", help="time only the QKV prologue (for profiling)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward leg")
    ap.add_argument("--fp8-only", action="store_true", help="time only the FP8 forward (for profiling)")
    ap.add_argument("--bwd-only", action="store_true", help="time only the backward (for profiling)")
    ap.add_argument("--no-gemm-ref", action="store_true", help="skip the library GEMM calibration")
    ap.add_argument("--no-legs", action="store_true", help="skip the forward legs on the other workloads")
    ap.add_argument("--gemm-ref-only", action="store_true", help="time only the library GEMM calibration")
    ap.add_argument("--split", default="auto",
                    help="'auto': lsv_attn_fwd_tail (the last, partial round of query tiles cut into key ranges "
                         "when that plan cuts any, else lsv_attn_fwd); or a number of key ranges for every tile "
                         "(lsv_attn_fwd_split; 1 = lsv_attn_fwd)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward of one rank's share runs on a "
              "single MI355X and no cross-GPU path is built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    if args.copy_bytes > 0:
        copy_calibration(args.copy_bytes, args.steps)
        return

    import torch
    import long_sequence_video_amd as lsv
    if not os.path.exists(lsv.LIB_PATH):
        from long_sequence_video_amd.build import build
        build()
    if args.prologue_only:
        print(json.dumps({"qkv_prologue": bench_prologue(args.steps, args.warmup)}), flush=True)
        return
    if args.fp8_only:
        print(json.dumps({"attn_fwd_fp8": bench_fp8(args.config, args.steps, args.warmup, args.split)}),
              flush=True)
        return
    if args.bwd_only:
        print(json.dumps({"attn_bwd": bench_backward(args.config, args.steps, args.warmup)}), flush=True)
        return
    if args.gemm_ref_only:
        print(json.dumps({"mfma_reference": bench_gemm_reference("bf16", max(args.steps, 10), args.warmup),
                          "mfma_reference_fp8": bench_gemm_reference("fp8", max(args.steps, 10), args.warmup)}),
              flush=True)
        return

    t0 = time.perf_counter()
    inp = make_inputs(args.config)
    log(f"generated {args.config}: {inp.total_tokens} tokens x {inp.n_heads} heads in {time.perf_counter() - t0:.1f} s")
    flops = inp.flops()
    ms_per_step, per_step, n_split = time_forward(inp, args.steps, args.warmup, args.split)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"{args.config}: {ms_per_step:.3f} ms/step, {tflops:.1f} TFLOP/s, {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak")

    peak_at_clock, cus, khz = lsv.lsv_device_peak(0)
    executed = None
    if isinstance(n_split, dict):
        kernel = "attn_fwd_tail_kernel"
        traffic, traffic_src = measured_traffic(inp.name, kernel="attn_fwd_tail")
        executed = measured_mfma_flops(inp.name, KERNEL_SOURCE, "attn_fwd_tail")
    elif n_split == 1:
        kernel = "attn_fwd_tail_kernel (nothing cut)"   # what lsv_attn_fwd launches
        traffic, traffic_src = measured_traffic(inp.name)
        executed = measured_mfma_flops(inp.name, KERNEL_SOURCE, "attn_fwd")
    else:
        kernel = "attn_fwd_split_kernel + attn_fwd_combine_kernel"
        traffic, traffic_src = None, "not measured for the key-split launch"
    # HBM-minimal bytes per launch: q, k, v read once, O written once (bf16), LSE (fp32).
    algorithmic_bytes = 4 * inp.total_tokens * inp.n_heads * inp.head_dim * 2 + inp.total_tokens * inp.n_heads * 4
    result = {
        "metric": "BF16 attn fwd TFLOP/s (4*S^2*H*D), 56h x 128d, 19k-104k tok; % MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) bf16 q/k/v; no dataset)",
        "config": {
            "workload": inp.name,
            "seqlens": inp.seqlens,
            "tokens": inp.total_tokens,
            "heads": inp.n_heads,
            "head_dim": inp.head_dim,
            "causal": False,
            "flops_per_step": flops,
            "parallelism": "single GPU",
            "key_split": n_split,
        },
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms": {"p50": round(float(np.percentile(per_step, 50)), 4),
                    "p95": round(float(np.percentile(per_step, 95)), 4),
                    "min": round(per_step[0], 4), "max": round(per_step[-1], 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch",
            "traffic_source": traffic_src,
            "algorithmic_hbm_bytes": algorithmic_bytes,
            "kernel": kernel,
            # SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 from the same counter summary: the counted flops
            # plus the masked padding of partial tiles
            "mfma_flops_executed": executed,
            "peak_at_reported_clock": round(peak_at_clock, 1),
            "compute_units": cus,
            "clock_mhz": khz // 1000,
        },
    }
    if not args.no_legs:
        result["forward_legs"] = [bench_forward_leg(name, args.split) for name in FORWARD_LEGS
                                  if name != args.config]
        by_name = {leg["workload"]: leg for leg in result["forward_legs"]}
        if "fallback_s38000_h56" in by_name and "h3_s38000_h56" in by_name:
            # what a workload pays when every workgroup reruns on the exact path
            by_name["fallback_s38000_h56"]["vs_fast_path"] = round(
                by_name["fallback_s38000_h56"]["ms_per_step"] / by_name["h3_s38000_h56"]["ms_per_step"], 3)
    if not args.no_fp8:
        result["attn_fwd_fp8"] = bench_fp8(args.config, min(max(args.steps, 3), 10), max(min(args.warmup, 2), 1),
                                           args.split)
        if not args.no_legs and args.config != FP8_LEG:
            # one sp=4 rank's share: the launch whose last round the tail split fills
            result["attn_fwd_fp8"]["legs"] = [bench_fp8(FP8_LEG, 100, 20, args.split)]
        if not args.no_gemm_ref:
            ref8 = bench_gemm_reference("fp8", steps=64)
            result["attn_fwd_fp8"]["mfma_reference"] = ref8
            result["attn_fwd_fp8"]["vs_library_gemm"] = round(result["attn_fwd_fp8"]["roofline"]["achieved"] /
                                                              ref8["tflops"], 4)
    if not args.no_bwd:
        result["attn_bwd"] = bench_backward(args.config, min(max(args.steps, 3), 5), max(min(args.warmup, 2), 1))
    if not args.no_prologue:
        result["qkv_prologue"] = bench_prologue(max(args.steps, 10), max(args.warmup, 2))
        result["qkv_prologue_fused_q"] = bench_qnorm(min(max(args.steps, 3), 5), 1)
    if not args.no_gemm_ref:
        ref = bench_gemm_reference("bf16")
        result["mfma_reference"] = ref
        result["vs_library_gemm"] = round(tflops / ref["tflops"], 4)
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(inp)
        log(f"cpu baseline: {result['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s "
            f"({time.perf_counter() - t0:.1f} s incl. calibration)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
