"""GPU parity of the FP8 (e4m3) forward that cuts the last, partial round's query tiles into key
ranges (``lsv_attn_fwd_fp8_tail``) against the fp64 FP8 oracle, through the C ABI.

Same bars as the FP8 forward (``tests/test_fp8_gpu.py``, derived from the simulation of the
kernel's own arithmetic). A cut tile's ranges each round their weights to e4m3 against their own
running max, and the merge is fp32, so cut rows differ from ``lsv_attn_fwd_fp8``'s by rounding
only; the tiles of the whole rounds are computed exactly as ``lsv_attn_fwd_fp8`` computes them and
must be bit-identical to it. The plans are ``lsv_attn_fwd_tail_plan``'s (256-row query tiles, as
in the BF16 forward); small packs take small ``compute_units`` values so that they cut 2-8 ranges,
and the 19,394 x 14 share, the 38,000 x 14 share and the 161,394-token pack run with the device's
own count.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from tests.gpu_common import run_fp8_tail, sample_rows, say, whole_tile_rows
from tests.test_fp8_gpu import compare_fp8

pytestmark = pytest.mark.gpu


def check_whole_tiles(out, lse, ref_o, ref_l, whole):
    assert np.array_equal(out[whole], ref_o[whole])
    assert np.array_equal(lse.T[whole].view(np.uint32), ref_l.T[whole].view(np.uint32))


@pytest.mark.parametrize("seqlens,heads,units", [
    ([5000], 8, 128),            # 20 tiles per XCD: the last 4 of each (one head's, ragged last), 4 ranges
    ([8200], 8, 64),             # 33 per XCD: each head's last tile (8 rows), 8 ranges
    ([9000, 300, 4097], 2, 96),  # 27 per XCD: 24 tail tiles, 12 of them empty, 4 ranges
    ([9000, 300], 4, 256),       # 36 per XCD: 32 tail tiles (16 empty, 4 ragged), 8 ranges
    ([1, 5000], 1, 256),         # 5 per XCD, all cut: no whole tile; the 1-token segment's ranges 2-4 are empty
    ([2048, 300], 1, 256),       # 2 per XCD, all cut: 2 ranges, the 300-token segment's tiles among them
    ([4000, 4000], 1, 128),      # 4 per XCD: 3 ranges of 1,344, 1,344 and 1,312 keys
    ([5000], 7, 128),            # 140 tiles, 18 per XCD, the last 2 cut in 4 ranges; XCD 7's last 4 do not exist
    ([4104], 7, 96),             # 119 tiles, 15 per XCD, the last 3 cut in 4 ranges; XCD 7's last one does not exist
    ([3590, 1200], 1, 128),      # 30 tiles, 4 per XCD, all cut in 3 ranges; XCD 7's last 2 do not exist
])
def test_fp8_tail_all_rows(gpu, seqlens, heads, units):
    f8 = gen.quantize_fp8(gen.generate(seqlens, heads, seed=900 + len(seqlens) + units, name="fp8_tail"))
    whole, split, n_tail = whole_tile_rows(f8, units)
    assert split > 1 and n_tail > 0
    say(f"case fp8 tail {seqlens} h{heads} units {units}: {n_tail} tail tiles x {split} ranges")
    out, lse, ref_o, ref_l = run_fp8_tail(f8, gpu, units)
    check_whole_tiles(out, lse, ref_o, ref_l, whole)
    compare_fp8(f8, out, lse, label=f"fp8 tail {seqlens} h{heads} units {units}")


def test_fp8_tail_late_dominant_key_in_a_later_range(gpu):
    """Every tile cut into 4 ranges (1,280 keys but the last); query row 9 meets a key in the third range that
    dominates its row by about 53 log2 units (the construction of the FP8 dominant-key test): that
    range's running max is raised, its LSE dominates the merge by ~2^-47, and the row's O equals
    bf16(fp32(dv * v8_j)) bit for bit, as in the plain kernel."""
    f8 = gen.quantize_fp8(gen.generate([5000], 2, seed=953, name="fp8_tail_dom"))
    i, j = 9, 2900
    rng = np.random.default_rng(53)
    q120, k240 = gen.f64_to_e4m3_bits(np.array([120.0, 240.0]))
    for h in range(2):
        neg = rng.random(128) < 0.5
        f8.q[i, h] = np.where(neg, q120 | 0x80, q120)
        f8.k[j, h] = np.where(neg, k240 | 0x80, k240)
        # no zero in v_j: the other ranges' weights (~1e-13 after the merge) then stay below half
        # an fp32 ulp of every O element, which is what makes the merged row exact
        f8.v[j, h] = np.where((f8.v[j, h] & 0x7F) == 0, 0x08, f8.v[j, h])
    whole, split, n_tail = whole_tile_rows(f8, 256)
    assert split == 4 and not whole.any()  # 40 tiles, 5 per XCD of 32 slots: all cut
    say(f"case fp8 tail dominant key: {n_tail} tail tiles x {split} ranges")
    out, lse, ref_o, _ = run_fp8_tail(f8, gpu, 256)
    from oracle import e4m3_bits_to_f64
    for h in range(2):
        want_o = gen.f64_to_bf16_bits(np.float32(f8.descale_v) * e4m3_bits_to_f64(f8.v[j, h]).astype(np.float32))
        assert np.array_equal(out[i, h], want_o), h
        assert np.array_equal(out[i, h], ref_o[i, h]), h
    compare_fp8(f8, out, lse, label="fp8 tail dominant key")


def test_fp8_tail_rows_outside_segments_untouched(gpu):
    """96 logical tiles on 88 units, 12 per XCD: the last of each is cut into 3 key ranges (4 of
    them empty tiles of the short segments, 2 the ragged last tile of a 4,000-token segment);
    NaN bytes outside every segment."""
    f8 = gen.quantize_fp8(gen.generate([61, 0, 4000], 2, seed=72, total_tokens=4100, name="fp8_tail_poison"))
    for t in (f8.q, f8.k, f8.v):
        t[4061:] = 0x7F  # e4m3 NaN outside every segment
    say("case fp8 tail poison")
    out, lse, _, _ = run_fp8_tail(f8, gpu, 88, out_fill=0x1234)
    assert np.all(out[4061:] == 0x1234) and np.all(lse[:, 4061:] == -7.0)
    compare_fp8(f8, out, lse, rows=np.arange(4061), label="fp8 tail poison")


@pytest.mark.parametrize("name", ["sp4_share_s19394_h14", "s4096_h56_kboost"])
def test_fp8_tail_workloads_every_row(gpu, name):
    """The benchmark's plans (the device's compute units): every row against the oracle, whole
    tiles bit-identical to lsv_attn_fwd_fp8, and two runs bit-identical. 19,394 x 14 cuts the
    last 5 tiles of each XCD into 6 ranges; 4,096 x 56 is left whole (half a round)."""
    import long_sequence_video_amd as lsv
    f8 = gen.make_fp8_config(name)
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(f8, units)
    say(f"case fp8 tail {name}: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_fp8_tail(f8, gpu)
    check_whole_tiles(out, lse, ref_o, ref_l, whole)
    out2, lse2, _, _ = run_fp8_tail(f8, gpu)
    assert np.array_equal(out, out2) and np.array_equal(lse.view(np.uint32), lse2.view(np.uint32))
    compare_fp8(f8, out, lse, label=f"fp8 tail {name}")


@pytest.mark.parametrize("name,seqlen,heads,seed", [
    ("fp8_sp4_share_s38000_h14", 38000, 14, 1008),    # 2,086 tiles (not a multiple of 8): 6 ranges
    ("fp8_varlen_19394_38000_104000_h56", None, 56, 1005),  # the pack: 24 tail tiles x 8 ranges
])
def test_fp8_tail_full_size_as_the_benchmark_launches_it(gpu, name, seqlen, heads, seed):
    """Full-size launches with the device's plan: whole tiles bit-identical to lsv_attn_fwd_fp8;
    every row of the cut tiles, the first and last 32 rows of every segment and random rows
    against the oracle, on every head."""
    import torch
    import long_sequence_video_amd as lsv
    if seqlen is None:
        f8 = gen.make_fp8_config("varlen_19394_38000_104000_h56")
    else:
        f8 = gen.quantize_fp8(gen.generate([seqlen], heads, seed=seed, rms_qk=True, name=name))
    units = lsv.lsv_device_peak(0)[1]
    whole, split, n_tail = whole_tile_rows(f8, units)
    assert split > 1 and n_tail > 0
    say(f"case fp8 tail {name}: {n_tail} tail tiles x {split} ranges on {units} compute units")
    out, lse, ref_o, ref_l = run_fp8_tail(f8, gpu)
    check_whole_tiles(out, lse, ref_o, ref_l, whole)
    del ref_o, ref_l
    cut = np.flatnonzero(~whole.all(axis=1))
    rows = np.union1d(cut, sample_rows(f8, 8, seed=15, tile=32))
    say(f"case fp8 tail {name}: oracle on {len(rows)} rows ({len(cut)} in cut tiles)")
    compare_fp8(f8, out, lse, rows=rows, label=f"fp8 tail {name}")
    del f8, out, lse
    torch.cuda.empty_cache()
