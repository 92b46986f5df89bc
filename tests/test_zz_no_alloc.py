"""The backward's no-allocation entry point, lsv_attn_bwd_noalloc, against lsv_attn_bwd.

Both run the same two kernels; the no-alloc one keeps the per-(head, token) statistics in
the library's own device scratch instead of a caller's workspace. Two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents, which the second
must overwrite where it reads): each must give gradients bit-identical to lsv_attn_bwd's on
the same inputs and match the fp64 oracle at the backward's bar. The first call runs on the
null stream, the second on a side stream (the scratch is looked up through the stream's
device).
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import attention_fp64
from tests.gpu_common import from_dev, say, to_dev
from tests.test_bwd_gpu import compare as compare_bwd

pytestmark = pytest.mark.gpu


def _case(seqlens, heads, seed, device, side):
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate(seqlens, heads, seed=seed, name="noalloc")
    o, l, _ = attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale)
    do = gen.normal_bf16(inp.q.size, seed + 1, 9).reshape(inp.q.shape)
    q, k, v, o_d, do_d = (to_dev(x, device) for x in (inp.q, inp.k, inp.v, gen.f64_to_bf16_bits(o), do))
    lse_d = torch.from_numpy(l.astype(np.float32)).to(device)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    ref = lsv.attn_bwd(q, k, v, o_d, do_d, lse_d, cu, inp.max_seqlen, inp.scale)
    torch.cuda.synchronize(device)
    ref = tuple(from_dev(g) for g in ref)
    grads = [torch.full_like(q, 7.0) for _ in range(3)]
    stream = None
    if side:
        stream = torch.cuda.Stream(device=device)
        stream.wait_stream(torch.cuda.current_stream(device))
    lsv.attn_bwd_noalloc(q, k, v, o_d, do_d, lse_d, cu, inp.max_seqlen, inp.scale, dq=grads[0], dk=grads[1],
                         dv=grads[2], stream=stream)
    torch.cuda.synchronize(device)
    got = tuple(from_dev(g) for g in grads)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert np.array_equal(a, b), name
    compare_bwd(inp, do, got, label=f"noalloc {seqlens} h{heads}")


def test_noalloc_matches_workspace_entry_two_calls(gpu):
    say("case noalloc: first call, 2 segments x 3 heads, null stream")
    _case([1000, 700], 3, 951, gpu, side=False)
    say("case noalloc: second call, smaller, side stream")
    _case([300, 77], 2, 953, gpu, side=True)

