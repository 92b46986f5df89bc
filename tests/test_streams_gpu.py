"""The torch conveniences on a stream other than the current one.

The binding allocates outputs and workspaces with torch's caching allocator on the current
stream while the kernels run on the given stream. Each such buffer must stay reserved for
that stream's work: right after each call this test allocates and fills a buffer of the
workspace's size on the current stream, the allocation that would get a workspace the
binding had already released, and the results must still match the oracle.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import attention_fp64
from tests.gpu_common import compare, from_dev, say, to_dev
from tests.test_bwd_gpu import compare as compare_bwd

pytestmark = pytest.mark.gpu


def _setup(inp, device):
    import torch
    q, k, v = (to_dev(x, device) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    side = torch.cuda.Stream(device=device)
    side.wait_stream(torch.cuda.current_stream(device))
    return q, k, v, cu, side


def _reuse(nbytes, device):
    """Allocate and overwrite nbytes on the current stream."""
    import torch
    junk = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    junk.fill_(0xFF)
    return junk


def test_split_forward_on_a_side_stream(gpu):
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate([1500, 700], 2, seed=901, name="side_split")
    q, k, v, cu, side = _setup(inp, gpu)
    say("case split forward on a side stream")
    out, lse = lsv.attn_fwd_split(q, k, v, cu, inp.max_seqlen, inp.scale, 3, stream=side)
    junk = _reuse(lsv.lsv_attn_fwd_split_workspace_size(inp.total_tokens, inp.n_heads, 3), gpu)
    side.synchronize()
    torch.cuda.synchronize(gpu)
    del junk
    compare(inp, from_dev(out), lse.cpu().numpy(), label="split on a side stream")


def test_forward_and_backward_on_a_side_stream(gpu):
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate([900, 333], 2, seed=902, name="side_bwd")
    q, k, v, cu, side = _setup(inp, gpu)
    say("case forward + backward on a side stream")
    out, lse = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale, stream=side)
    side.synchronize()
    compare(inp, from_dev(out), lse.cpu().numpy(), label="forward on a side stream")
    # the backward is handed the oracle's O / LSE, as in the backward parity tests
    o, l, _ = attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale)
    o_d = to_dev(gen.f64_to_bf16_bits(o), gpu)
    lse_d = torch.from_numpy(l.astype(np.float32)).to(gpu)
    do = gen.normal_bf16(inp.q.size, 903, 9).reshape(inp.q.shape)
    do_d = to_dev(do, gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    grads = lsv.attn_bwd(q, k, v, o_d, do_d, lse_d, cu, inp.max_seqlen, inp.scale, stream=side)
    junk = _reuse(lsv.lsv_attn_bwd_workspace_size(inp.total_tokens, inp.n_heads), gpu)
    side.synchronize()
    torch.cuda.synchronize(gpu)
    del junk
    compare_bwd(inp, do, tuple(from_dev(g) for g in grads), label="backward on a side stream")
