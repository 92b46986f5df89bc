"""Head counts other than the workloads' 56 and 14: 1, 3 and 112 heads (row strides of 256 B,
768 B and 28,672 B; the logical tiles are head-major, so the head count also sets how each XCD's
range of tiles falls across heads). Every row of the BF16 forward (``lsv_attn_fwd`` and
``lsv_attn_fwd_tail`` with a compute-unit count whose plan cuts tiles that hold rows), of the FP8
tail forward and of the backward against the oracles; whole tail tiles bit-identical to the plain
launch."""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from tests.gpu_common import compare, from_dev, run_fp8_tail, say, to_dev, whole_tile_rows

pytestmark = pytest.mark.gpu

CASES = [([3000, 77, 5000], 1), ([1000, 2500], 3), ([2000, 3000], 112)]


def _cutting_units(inp):
    """The smallest compute-unit count (a multiple of 8) whose tail plan cuts query tiles that
    hold rows, or None."""
    for units in range(16, 1025, 8):
        whole, split, n_tail = whole_tile_rows(inp, units)
        if split > 1 and n_tail > 0 and not whole.all():
            return units
    return None


@pytest.mark.parametrize("seqlens,heads", CASES)
def test_head_counts_forward_fp8_and_backward(gpu, seqlens, heads):
    import torch
    import long_sequence_video_amd as lsv
    from tests.test_bwd_gpu import _dout, compare as compare_bwd, run_bwd
    from tests.test_fp8_gpu import compare_fp8
    inp = gen.generate(seqlens, heads, seed=90 + heads, name=f"h{heads}")
    units = _cutting_units(inp)
    say(f"case {heads} heads {seqlens}: tail plan on {units} units")
    q, k, v = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(gpu)
    o1, l1 = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale)
    torch.cuda.synchronize(gpu)
    o1, l1 = from_dev(o1), l1.cpu().numpy()
    compare(inp, o1, l1, label=f"h{heads} lsv_attn_fwd")
    if units is not None:
        whole, split, n_tail = whole_tile_rows(inp, units)
        o2, l2 = lsv.attn_fwd_tail(q, k, v, cu, inp.max_seqlen, inp.scale, compute_units=units)
        torch.cuda.synchronize(gpu)
        o2, l2 = from_dev(o2), l2.cpu().numpy()
        assert np.array_equal(o2[whole], o1[whole])
        assert np.array_equal(l2.T[whole].view(np.uint32), l1.T[whole].view(np.uint32))
        compare(inp, o2, l2, label=f"h{heads} lsv_attn_fwd_tail ({n_tail} tiles x {split})")
        f8 = gen.quantize_fp8(inp)
        out, lse, ref_o, ref_l = run_fp8_tail(f8, gpu, units)
        assert np.array_equal(out[whole], ref_o[whole])
        compare_fp8(f8, out, lse, label=f"h{heads} fp8 tail")
    del q, k, v
    do = _dout(inp, 90 + heads)
    grads = run_bwd(inp, do, gpu)
    compare_bwd(inp, do, grads, label=f"h{heads} bwd")
    torch.cuda.empty_cache()
