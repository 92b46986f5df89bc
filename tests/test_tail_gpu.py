"""GPU parity of the forward that cuts the last, partial round's query tiles into key ranges
(``lsv_attn_fwd_tail``) against the fp64 oracle, through the C ABI.

Same tolerances as the forward (bf16 O max-abs 2e-2, mean-abs 2e-3; LSE max-abs 1e-3). The
tiles of the whole rounds are computed exactly as ``lsv_attn_fwd`` computes them, so their rows
must be bit-identical to it; every row of the cut tiles is checked against the oracle. Small
packs take small ``compute_units`` values so that their plans cut 2-8 ranges (including tail
tiles that are empty or ragged, segments shorter than a range, and a pack with no whole tile);
the 19,394 x 14 workload (cut) and the 4,096 x 56 one (left whole: its last round is half full)
run with the device's own count, the plans the benchmark times.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from tests.gpu_common import compare, from_dev, sample_rows, say, to_dev, whole_tile_rows

pytestmark = pytest.mark.gpu


def run_tail(inp, device, units=None, *, out_fill=None):
    import torch
    import long_sequence_video_amd as lsv
    q, k, v = (to_dev(x, device) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    out = torch.empty_like(q)
    lse = torch.empty((inp.n_heads, inp.total_tokens), dtype=torch.float32, device=device)
    if out_fill is not None:
        out.view(torch.int16).fill_(int(np.int16(np.uint16(out_fill))))
        lse.fill_(-7.0)
    lsv.attn_fwd_tail(q, k, v, cu, inp.max_seqlen, inp.scale, compute_units=units, out=out, lse=lse)
    ref_o, ref_l = lsv.attn_fwd(q, k, v, cu, inp.max_seqlen, inp.scale)
    torch.cuda.synchronize(device)
    return from_dev(out), lse.cpu().numpy(), from_dev(ref_o), ref_l.cpu().numpy()


@pytest.mark.parametrize("seqlens,heads,units", [
    ([5000], 8, 128),            # 20 tiles per XCD: the last 4 of each (one head's, ragged last), 4 ranges
    ([8200], 8, 64),             # 33 per XCD: each head's last tile (8 rows), 8 ranges
    ([9000, 300, 4097], 2, 96),  # 27 per XCD: 24 tail tiles, 12 of them empty, 4 ranges
    ([9000, 300], 4, 256),       # 36 per XCD: 32 tail tiles (16 empty, 4 ragged), 8 ranges
    ([1, 5000], 1, 256),         # 5 per XCD, all cut: no whole tile; the 1-token segment's ranges 2-4 are empty
    ([2048, 300], 1, 256),       # 2 per XCD, all cut: 2 ranges, the 300-token segment's tiles among them
    ([4000, 4000], 1, 128),      # 4 per XCD: 3 ranges
    # query tiles not a multiple of 8: the last XCD's range runs past the end
    ([5000], 7, 128),            # 140 tiles, 18 per XCD, the last 2 cut in 4 ranges; XCD 7's last 4 do not exist
    ([4104], 7, 96),             # 119 tiles, 15 per XCD, the last 3 cut in 4 ranges; XCD 7's last one does not exist
    ([3590, 1200], 1, 128),      # 30 tiles, 4 per XCD, all cut in 3 ranges; XCD 7's last 2 do not exist
])
def test_tail_all_rows(gpu, seqlens, heads, units):
    inp = gen.generate(seqlens, heads, seed=800 + len(seqlens) + units, name="tail")
    whole, split, n_tail = whole_tile_rows(inp, units)
    assert split > 1 and n_tail > 0
    say(f"case tail {seqlens} h{heads} units {units}: {n_tail} tail tiles x {split} ranges")
    out, lse, ref_o, ref_l = run_tail(inp, gpu, units)
    assert np.array_equal(out[whole], ref_o[whole])
    assert np.array_equal(lse.T[whole].view(np.uint32), ref_l.T[whole].view(np.uint32))
    compare(inp, out, lse, label=f"tail {seqlens} h{heads} units {units}")


def test_tail_rows_outside_segments_untouched(gpu):
    """96 logical tiles on 88 units, 12 per XCD: the last of each is cut into 3 key ranges (4 of
    them empty tiles of the short segments, 2 the ragged last tile of a 4,000-token segment);
    NaN outside every segment."""
    inp = gen.generate([61, 0, 4000], 2, seed=71, total_tokens=4100, name="tail_poison")
    for t in (inp.q, inp.k, inp.v):
        t[4061:] = 0x7FC0  # NaN outside every segment
    say("case tail poison")
    out, lse, _, _ = run_tail(inp, gpu, 88, out_fill=0x1234)
    assert np.all(out[4061:] == 0x1234) and np.all(lse[:, 4061:] == -7.0)
    compare(inp, out, lse, rows=np.arange(4061), label="tail poison")


@pytest.mark.parametrize("name", ["sp4_share_s19394_h14", "s4096_h56_kboost"])
def test_tail_workloads_every_row(gpu, name):
    """The benchmark's plans (the device's compute units): every row against the oracle, whole
    tiles bit-identical to lsv_attn_fwd, and two runs bit-identical."""
    import long_sequence_video_amd as lsv
    inp = gen.make_config(name)
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(inp, units)
    say(f"case tail {name}: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_tail(inp, gpu)
    assert np.array_equal(out[whole], ref_o[whole])
    out2, lse2, _, _ = run_tail(inp, gpu)
    assert np.array_equal(out, out2) and np.array_equal(lse.view(np.uint32), lse2.view(np.uint32))
    compare(inp, out, lse, label=f"tail {name}")


@pytest.mark.parametrize("name", ["varlen_19394_38000_104000_h56", "h56_s104000"])
def test_tail_full_size_as_the_benchmark_launches_it(gpu, name):
    """The 161,394-token pack and its 104,000-token segment alone, in the launch the benchmark
    times (the device's compute units): whole tiles bit-identical to lsv_attn_fwd; every row of
    the cut tiles (the last tiles of a head in each XCD's range) plus the first and last tiles of
    every segment and random rows against the oracle, on every head."""
    import torch
    import long_sequence_video_amd as lsv
    if name == "h56_s104000":
        inp = gen.generate([104000], 56, seed=1005, name=name)
    else:
        inp = gen.make_config(name)
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(inp, units)
    assert split > 1 and n_tail > 0
    say(f"case tail {name}: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_tail(inp, gpu)
    assert np.array_equal(out[whole], ref_o[whole])
    assert np.array_equal(lse.T[whole].view(np.uint32), ref_l.T[whole].view(np.uint32))
    del ref_o, ref_l
    cut = np.flatnonzero(~whole.all(axis=1))
    rows = np.union1d(cut, sample_rows(inp, 16, seed=12, tile=32))
    say(f"case tail {name}: oracle on {len(rows)} rows ({len(cut)} in cut tiles)")
    compare(inp, out, lse, rows=rows, label=f"tail {name}")
    del inp, out, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,seqlen,seed", [("sp4_share_s38000_h14", 38000, 1008),
                                               ("sp4_share_s104000_h14", 104000, 1009)])
def test_tail_sp4_shares_with_a_ragged_xcd_range(gpu, name, seqlen, seed):
    """One sp=4 rank's 14-head share of the 38,000- and 104,000-token clips (RMS-normalised Q/K):
    2,086 and 5,698 query tiles, not multiples of 8, so the last XCD's range runs past the end.
    On 256 compute units 38,000 x 14 cuts the last 5 tiles of each XCD into 6 ranges, and
    104,000 x 14 (9 tiles past its last round) runs whole, as lsv_attn_fwd. Whole tiles
    bit-identical to lsv_attn_fwd; every cut-tile row, the first and last tiles of every
    segment and random rows against the oracle, on every head."""
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate([seqlen], 14, seed=seed, rms_qk=True, name=name)
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(inp, units)
    assert ((seqlen + 255) // 256 * 14) % 8 != 0
    say(f"case tail {name}: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_tail(inp, gpu)
    assert np.array_equal(out[whole], ref_o[whole])
    assert np.array_equal(lse.T[whole].view(np.uint32), ref_l.T[whole].view(np.uint32))
    del ref_o, ref_l
    cut = np.flatnonzero(~whole.all(axis=1))
    rows = np.union1d(cut, sample_rows(inp, 16, seed=14, tile=32))
    say(f"case tail {name}: oracle on {len(rows)} rows ({len(cut)} in cut tiles)")
    compare(inp, out, lse, rows=rows, label=f"tail {name}")
    del inp, out, lse
    torch.cuda.empty_cache()


def test_tail_at_the_largest_supported_segment(gpu):
    """299,593 x 56, the largest segment the 32-bit in-segment offsets allow, with the device's
    plan (the last 5 tiles of one head per XCD cut into 6 ranges, so the cut ranges start deep
    into the segment): whole tiles bit-identical to lsv_attn_fwd, every cut-tile row and the
    first and last tiles against the oracle."""
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate([299_593], 56, seed=1006, name="max_segment_s299593_h56")
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(inp, units)
    say(f"case tail max segment: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_tail(inp, gpu)
    assert np.array_equal(out[whole], ref_o[whole])
    assert np.array_equal(lse.T[whole].view(np.uint32), ref_l.T[whole].view(np.uint32))
    del ref_o, ref_l
    if n_tail:
        cut = np.flatnonzero(~whole.all(axis=1))
        rows = np.union1d(cut, sample_rows(inp, 4, seed=13, tile=32))
        compare(inp, out, lse, rows=rows, label="tail max segment")
    del inp, out, lse
    torch.cuda.empty_cache()
