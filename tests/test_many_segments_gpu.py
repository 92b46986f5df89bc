"""A pack of many clips: 1,000 segments of 0 to 500 tokens plus two of 3,000 and 5,000 tokens, 4
heads. The grid is then 20 query tiles x 1,002 segments x 4 heads = 80,160 logical tiles, most of
them past their segment's end (they exit at once), and each XCD's range crosses hundreds of
segments. Every row of the BF16 forward (``lsv_attn_fwd``, and ``lsv_attn_fwd_tail`` with a
compute-unit count whose plan cuts tiles that hold rows), the FP8 tail forward and the backward is
checked against the oracles; the tail launch's whole tiles are bit-identical to
``lsv_attn_fwd``'s."""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from tests.gpu_common import compare, from_dev, run_fp8_tail, say, to_dev, whole_tile_rows

pytestmark = pytest.mark.gpu


def _pack():
    rng = np.random.default_rng(2024)
    lens = [int(x) for x in rng.integers(0, 501, size=1000)]
    lens[300:300] = [3000]
    lens[700:700] = [5000]
    return gen.generate(lens, 4, seed=77, name="many_segments")


def _cutting_units(inp):
    """The smallest compute-unit count (a multiple of 8) whose tail plan cuts query tiles that
    hold rows (most tiles of this grid lie past their segment's end)."""
    for units in range(64, 1025, 8):
        whole, split, n_tail = whole_tile_rows(inp, units)
        if split > 1 and n_tail > 0 and not whole.all():
            return units
    raise AssertionError("no compute-unit count in 64..1024 cuts a tile that holds rows")


def test_many_segments_forward_plain_and_tail(gpu):
    import torch
    import long_sequence_video_amd as lsv
    inp = _pack()
    units = _cutting_units(inp)
    whole, split, n_tail = whole_tile_rows(inp, units)
    say(f"case many segments: {len(inp.cu_seqlens) - 1} segments, {inp.total_tokens} tokens, "
        f"tail plan {n_tail} tiles x {split} ranges on {units} units")
    q, k, v = (to_dev(x, gpu) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(gpu)
    o1, l1 = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale)
    o2, l2 = lsv.attn_fwd_tail(q, k, v, cu, inp.max_seqlen, inp.scale, compute_units=units)
    torch.cuda.synchronize(gpu)
    o1, l1, o2, l2 = from_dev(o1), l1.cpu().numpy(), from_dev(o2), l2.cpu().numpy()
    assert np.array_equal(o2[whole], o1[whole])
    assert np.array_equal(l2.T[whole].view(np.uint32), l1.T[whole].view(np.uint32))
    compare(inp, o1, l1, label="many segments lsv_attn_fwd")
    compare(inp, o2, l2, label="many segments lsv_attn_fwd_tail")


def test_many_segments_fp8_tail(gpu):
    from tests.test_fp8_gpu import compare_fp8
    inp = _pack()
    units = _cutting_units(inp)
    f8 = gen.quantize_fp8(inp)
    whole, _, _ = whole_tile_rows(inp, units)
    out, lse, ref_o, ref_l = run_fp8_tail(f8, gpu, units)
    assert np.array_equal(out[whole], ref_o[whole])
    compare_fp8(f8, out, lse, label="many segments fp8 tail")
    compare_fp8(f8, ref_o, ref_l, label="many segments fp8")


def test_many_segments_backward(gpu):
    from tests.test_bwd_gpu import _dout, compare as compare_bwd, run_bwd
    inp = _pack()
    do = _dout(inp, 2024)
    grads = run_bwd(inp, do, gpu)
    compare_bwd(inp, do, grads, label="many segments bwd")
