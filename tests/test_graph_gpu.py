"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph), through the C ABI.

One graph holds a forward step and a backward step the way a training or serving loop would
capture them: the K-side prologue and the forward with Q's norm and rotation in its Q load
(lsv_norm_rope, lsv_attn_fwd_qnorm, and lsv_attn_fwd_qnorm_tail), the tail-split forward
(lsv_attn_fwd_tail), the backward that allocates nothing (lsv_attn_bwd_noalloc) and the FP8
forward (lsv_attn_fwd_fp8, and lsv_attn_fwd_fp8_tail); the three tail launches share one
workspace, which their order on the stream makes safe. Every
buffer is allocated before capture and max_seqlen is passed, so nothing allocates, copies to
the host or synchronises inside the capture. The graph is replayed several times, with other
work and synchronisations between the replays, new inputs copied into the captured buffers in
between, and the outputs poisoned before each replay; every replay must be bit-identical to
the same calls made eagerly.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

SEQLENS = [5000, 0, 1200]
HEADS = 8
UNITS = 232   # a plan that cuts: 480 query tiles, 60 per XCD on 29 slots, the last 2 of each cut


def _host_inputs(seed, like=None):
    """(qnorm inputs, dO, e4m3 inputs). The e4m3 bytes of a second set reuse the first set's
    descales: the graph holds the descales it was captured with, as kernel arguments."""
    inp = gen.generate_qnorm(SEQLENS, HEADS, 96, seed=seed, name="graph")
    do = gen.normal_bf16(inp.q.size, seed, 9).reshape(inp.q.shape)
    f8 = gen.quantize_fp8(gen.Inputs("graph_fp8", inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale))
    if like is not None:
        f8 = gen.Fp8Inputs(f8.name, *(gen.quantize_e4m3_bf16(getattr(inp, x), getattr(like, "descale_" + x))
                                      for x in "qkv"), like.descale_q, like.descale_k, like.descale_v,
                           f8.cu_seqlens, f8.scale)
    return inp, do, f8


class Buffers:
    """Device buffers of every input and output of the captured step."""

    def __init__(self, inp, f8, device):
        import torch
        t, h = inp.total_tokens, inp.n_heads
        bf = lambda: torch.empty((t, h, 128), dtype=torch.bfloat16, device=device)  # noqa: E731
        self.q, self.k, self.v, self.do = bf(), bf(), bf(), bf()
        self.qw = torch.empty(128, dtype=torch.bfloat16, device=device)
        self.kw = torch.empty_like(self.qw)
        self.cos = torch.empty((t, 96), dtype=torch.bfloat16, device=device)
        self.sin = torch.empty_like(self.cos)
        self.q8, self.k8, self.v8 = (torch.empty((t, h, 128), dtype=torch.uint8, device=device) for _ in range(3))
        self.cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
        self.kn, self.o_qn, self.o, self.o8, self.o_qt, self.o8t = bf(), bf(), bf(), bf(), bf(), bf()
        self.dq, self.dk, self.dv = bf(), bf(), bf()
        self.l_qn, self.l, self.l8, self.l_qt, self.l8t = (torch.empty((h, t), dtype=torch.float32, device=device)
                                                           for _ in range(5))
        import long_sequence_video_amd as lsv
        self.ws = torch.empty(lsv.lsv_attn_fwd_tail_workspace_size(UNITS), dtype=torch.uint8, device=device)
        self.outputs = (self.kn, self.o_qn, self.l_qn, self.o, self.l, self.dq, self.dk, self.dv, self.o8, self.l8,
                        self.o_qt, self.l_qt, self.o8t, self.l8t)

    def load(self, inp, do, f8):
        import torch

        def put(dst, bits):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).reshape(dst.shape))
        for dst, bits in ((self.q, inp.q), (self.k, inp.k), (self.v, inp.v), (self.do, do), (self.qw, inp.q_weight),
                          (self.kw, inp.k_weight), (self.cos, inp.cos), (self.sin, inp.sin)):
            put(dst, bits)
        for dst, b in ((self.q8, f8.q), (self.k8, f8.k), (self.v8, f8.v)):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(b)).reshape(dst.shape))
        self.f8 = f8

    def poison(self):
        for t in self.outputs:
            t.fill_(float("nan"))

    def snapshot(self):
        return [t.clone() for t in self.outputs]


def step(b, inp):
    """The captured work: both forward paths, the backward and the FP8 forward."""
    import long_sequence_video_amd as lsv
    ms = max(SEQLENS)
    lsv.norm_rope(b.k, b.kw, b.cos, b.sin, eps=inp.eps, out=b.kn)
    lsv.attn_fwd_qnorm(b.q, b.kn, b.v, b.qw, b.cos, b.sin, b.cu, ms, inp.scale, eps=inp.eps, out=b.o_qn, lse=b.l_qn)
    lsv.attn_fwd_tail(b.q, b.k, b.v, b.cu, ms, inp.scale, compute_units=UNITS, out=b.o, lse=b.l, workspace=b.ws)
    lsv.attn_bwd_noalloc(b.q, b.k, b.v, b.o, b.do, b.l, b.cu, ms, inp.scale, dq=b.dq, dk=b.dk, dv=b.dv)
    lsv.attn_fwd_fp8(b.q8, b.k8, b.v8, b.f8.descale_q, b.f8.descale_k, b.f8.descale_v, b.cu, ms, b.f8.scale,
                     out=b.o8, lse=b.l8)
    lsv.attn_fwd_qnorm(b.q, b.kn, b.v, b.qw, b.cos, b.sin, b.cu, ms, inp.scale, eps=inp.eps, out=b.o_qt, lse=b.l_qt,
                       compute_units=UNITS, workspace=b.ws)
    lsv.attn_fwd_fp8_tail(b.q8, b.k8, b.v8, b.f8.descale_q, b.f8.descale_k, b.f8.descale_v, b.cu, ms, b.f8.scale,
                          compute_units=UNITS, out=b.o8t, lse=b.l8t, workspace=b.ws)


def _same(a, b):
    """Bitwise equality of two lists of tensors."""
    import torch
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_replays_of_a_captured_step_equal_eager_calls(gpu):
    import torch
    import long_sequence_video_amd as lsv
    split, n_tail = lsv.lsv_attn_fwd_tail_plan(len(SEQLENS), max(SEQLENS), HEADS, UNITS)
    assert split > 1 and n_tail > 0   # the tail kernel and its combine are in the graph
    first = _host_inputs(501)
    host = [first, _host_inputs(502, like=first[2])]
    b = Buffers(host[0][0], host[0][2], gpu)

    eager = []
    for inp, do, f8 in host:
        b.load(inp, do, f8)
        b.poison()
        step(b, inp)
        torch.cuda.synchronize(gpu)
        eager.append(b.snapshot())
    assert not _same(eager[0], eager[1])

    say("case graph capture")
    b.load(*host[0])
    side = torch.cuda.Stream(gpu)   # capture on a side stream, as torch requires
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):   # one warm-up call on the capture stream
        step(b, host[0][0])
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize(gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(b, host[0][0])
    torch.cuda.synchronize(gpu)

    for replay, which in enumerate((0, 1, 0, 1)):
        inp, do, f8 = host[which]
        b.load(inp, do, f8)
        b.poison()
        junk = torch.randn(1 << 20, device=gpu).sum()   # eager work between replays
        torch.cuda.synchronize(gpu)
        say(f"case graph replay {replay} (inputs {which})")
        graph.replay()
        torch.cuda.synchronize(gpu)
        assert torch.isfinite(junk)
        got = b.snapshot()
        assert _same(got, eager[which]), f"replay {replay} differs from the eager step"
    del graph
    torch.cuda.empty_cache()
