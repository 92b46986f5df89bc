"""GPU parity of the forward with the QKV prologue's Q side fused into the Q-tile load
(``lsv_attn_fwd_qnorm``) and of the single-tensor prologue (``lsv_norm_rope``), through the C ABI.

* ``lsv_norm_rope`` against the prologue oracle on every element (one bf16 ulp plus a
  cancellation allowance, 2^-7 |ref| + 2^-16 sum|terms|, and 99.9% correctly rounded: the
  prologue's own bar), and bit-identical to ``lsv_qkv_prologue``'s
  Q and K planes of one sequence (the same kernel step).
* ``lsv_attn_fwd_qnorm`` bit-identical to the two-pass path ``lsv_norm_rope(q)`` then
  ``lsv_attn_fwd`` (it computes Q with the prologue's exact fp32 steps and summation order), on
  every rotary width the prologue supports.
* ``lsv_attn_fwd_qnorm_tail`` (the launch that cuts the last, partial round of query tiles into
  key ranges) bit-identical to ``lsv_norm_rope(q)`` then ``lsv_attn_fwd_tail`` with the same plan.
* ``lsv_attn_fwd_qnorm`` against the oracle composition: the prologue oracle's exact Q and K
  rounded to bf16, then the attention oracle, at the forward's tolerances (O max-abs 2e-2,
  mean-abs 2e-3, LSE 1e-3); every row of ragged packs, sampled rows of the 161,394-token pack
  with each segment's own RoPE positions.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import bf16_bits_to_f64, norm_rope_rows_fp64
from tests.gpu_common import compare, from_dev, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _oracle_rows(x_bits, w_bits, cos_bits, sin_bits, eps, chunk=4096):
    """The prologue oracle on [T, H, 128] with one table row per token: (exact, magnitudes),
    evaluated ``chunk`` tokens at a time on a thread pool (rows are independent)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    t, h, d = x_bits.shape
    out = np.empty((t, h, d))
    mag = np.empty((t, h, d))

    def run(a):
        b = min(a + chunk, t)
        rows = x_bits[a:b].reshape((b - a) * h, d)
        o, m = norm_rope_rows_fp64(rows, w_bits, np.repeat(cos_bits[a:b], h, axis=0),
                                   np.repeat(sin_bits[a:b], h, axis=0), eps)
        out[a:b], mag[a:b] = o.reshape(b - a, h, d), m.reshape(b - a, h, d)

    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(run, range(0, t, chunk)))
    return out, mag


def _dev_tables(inp, device):
    if inp.rotary_dim == 0:
        return None, None
    return to_dev(inp.cos, device), to_dev(inp.sin, device)


@pytest.mark.parametrize("rotary_dim", [0, 16, 32, 48, 96, 112, 128])
def test_norm_rope_every_element_and_equal_to_the_qkv_prologue(gpu, rotary_dim):
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate_qnorm([300, 77], 3, rotary_dim, seed=81 + rotary_dim, tables="normal")
    say(f"case norm_rope R={rotary_dim}")
    x, w = to_dev(inp.k, gpu), to_dev(inp.k_weight, gpu)
    cos, sin = _dev_tables(inp, gpu)
    got = from_dev(lsv.norm_rope(x, w, cos, sin, eps=inp.eps))
    ref, mag = _oracle_rows(inp.k, inp.k_weight, inp.cos, inp.sin, inp.eps)
    err = np.abs(bf16_bits_to_f64(got) - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 2.0 ** -16 * mag + 1e-30    # the prologue tests' bar
    assert (err <= bound).all(), float((err / bound).max())
    assert np.mean(got == gen.f64_to_bf16_bits(ref)) >= 0.999
    # the stacked prologue on the same rows (one sequence: its [S, R] table is the per-token one)
    q, v = to_dev(inp.q, gpu), to_dev(inp.v, gpu)
    qw = to_dev(inp.q_weight, gpu)
    st = from_dev(lsv.qkv_prologue(q, x, v, qw, w, cos, sin, eps=inp.eps))
    torch.cuda.synchronize(gpu)
    assert np.array_equal(st[1], got)
    assert np.array_equal(st[0], from_dev(lsv.norm_rope(q, qw, cos, sin, eps=inp.eps)))


def _fused_and_two_pass(inp, device, max_seqlen=None, units=None):
    """(O, LSE) of lsv_attn_fwd_qnorm and of lsv_norm_rope(q) -> lsv_attn_fwd, on the same k, v
    (with ``units``: lsv_attn_fwd_qnorm_tail and lsv_norm_rope(q) -> lsv_attn_fwd_tail on that many
    compute units); k is the prologue oracle's K rounded to bf16."""
    import torch
    import long_sequence_video_amd as lsv
    kref, _ = _oracle_rows(inp.k, inp.k_weight, inp.cos, inp.sin, inp.eps)
    k_bits = gen.f64_to_bf16_bits(kref)
    q, k, v = (to_dev(x, device) for x in (inp.q, k_bits, inp.v))
    qw = to_dev(inp.q_weight, device)
    cos, sin = _dev_tables(inp, device)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
    ms = inp.max_seqlen if max_seqlen is None else max_seqlen
    o1, l1 = lsv.attn_fwd_qnorm(q, k, v, qw, cos, sin, cu, ms, inp.scale, eps=inp.eps, compute_units=units)
    qn = lsv.norm_rope(q, qw, cos, sin, eps=inp.eps)
    if units is None:
        o2, l2 = lsv.attn_fwd(qn, k, v, cu, ms, inp.scale)
    else:
        o2, l2 = lsv.attn_fwd_tail(qn, k, v, cu, ms, inp.scale, compute_units=units)
    torch.cuda.synchronize(device)
    return (from_dev(o1), l1.cpu().numpy()), (from_dev(o2), l2.cpu().numpy()), k_bits


def _composition(inp, k_bits):
    """The oracle composition as an ``inputs.Inputs``: bf16 of the prologue oracle's exact Q, the
    given K bits, raw V."""
    qref, _ = _oracle_rows(inp.q, inp.q_weight, inp.cos, inp.sin, inp.eps)
    return gen.Inputs(inp.name, gen.f64_to_bf16_bits(qref), k_bits, inp.v, inp.cu_seqlens, inp.scale)


@pytest.mark.parametrize("rotary_dim", [0, 16, 48, 96, 128])
@pytest.mark.parametrize("seqlens,heads", [([1, 0, 33, 300, 64], 3), ([1000], 2), ([127, 128, 129], 2)])
def test_fused_equals_two_pass_and_matches_the_oracle(gpu, seqlens, heads, rotary_dim):
    inp = gen.generate_qnorm(seqlens, heads, rotary_dim, seed=90 + len(seqlens) + rotary_dim)
    say(f"case attn_fwd_qnorm {seqlens} h{heads} R={rotary_dim}")
    (o1, l1), (o2, l2), k_bits = _fused_and_two_pass(inp, gpu)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    compare(_composition(inp, k_bits), o1, l1, label=f"qnorm {seqlens} h{heads} R={rotary_dim}")


@pytest.mark.parametrize("rotary_dim", [0, 96])
@pytest.mark.parametrize("seqlens,heads,units", [
    ([5000], 8, 128),            # 20 tiles per XCD: the last 4 cut into 4 ranges
    ([9000, 300, 4097], 2, 96),  # 27 per XCD: 24 tail tiles, 12 of them empty, 4 ranges
    ([4104], 7, 96),             # 119 tiles, 15 per XCD: the last 3 cut; XCD 7's last one does not exist
])
def test_fused_tail_equals_two_pass_tail_and_matches_the_oracle(gpu, seqlens, heads, units, rotary_dim):
    """lsv_attn_fwd_qnorm_tail bit-identical to lsv_norm_rope(q) -> lsv_attn_fwd_tail with the same
    plan (the cut tiles included), whole tiles bit-identical to lsv_attn_fwd_qnorm, and every row
    against the oracle composition."""
    from tests.gpu_common import whole_tile_rows
    # RoPE tables, as in the other oracle comparisons of the fused forward: the oracle composition
    # rounds its exact Q to bf16 on its own, and random N(0,1) tables scale Q so far that one ulp
    # of it moves a score by centinats
    inp = gen.generate_qnorm(seqlens, heads, rotary_dim, seed=97 + units + rotary_dim)
    whole, split, n_tail = whole_tile_rows(inp, units)
    assert split > 1 and n_tail > 0
    say(f"case attn_fwd_qnorm_tail {seqlens} h{heads} units {units} R={rotary_dim}: {n_tail} x {split}")
    (o1, l1), (o2, l2), k_bits = _fused_and_two_pass(inp, gpu, units=units)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    (o3, l3), _, _ = _fused_and_two_pass(inp, gpu)
    assert np.array_equal(o1[whole], o3[whole])
    assert np.array_equal(l1.T[whole].view(np.uint32), l3.T[whole].view(np.uint32))
    compare(_composition(inp, k_bits), o1, l1, label=f"qnorm tail {seqlens} h{heads} units {units}")


def test_fused_rows_outside_segments_untouched(gpu):
    """Tokens past cu[-1] hold NaN in q, k, v and the tables; their outputs keep the sentinel."""
    import torch
    import long_sequence_video_amd as lsv
    inp = gen.generate_qnorm([100, 0, 61], 2, 96, seed=95)
    pad = 39
    q, k, v = (np.concatenate([x, np.full((pad,) + x.shape[1:], 0x7FC0, np.uint16)]) for x in (inp.q, inp.k, inp.v))
    cos, sin = (np.concatenate([x, np.full((pad, 96), 0x7FC0, np.uint16)]) for x in (inp.cos, inp.sin))
    say("case attn_fwd_qnorm poison")
    out = torch.full((200, 2, 128), 3.0, dtype=torch.bfloat16, device=gpu)
    lse = torch.full((2, 200), -7.0, device=gpu)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(gpu)
    lsv.attn_fwd_qnorm(to_dev(q, gpu), to_dev(k, gpu), to_dev(v, gpu), to_dev(inp.q_weight, gpu), to_dev(cos, gpu),
                       to_dev(sin, gpu), cu, inp.max_seqlen, inp.scale, eps=inp.eps, out=out, lse=lse)
    torch.cuda.synchronize(gpu)
    o, l = from_dev(out), lse.cpu().numpy()
    assert np.all(bf16_bits_to_f64(o[161:]) == 3.0) and np.all(l[:, 161:] == -7.0)
    comp = _composition(inp, k[:161])
    compare(comp, o[:161], l[:, :161], label="qnorm poison")


def test_fused_varlen_pack_sampled(gpu):
    """The 161,394-token pack x 56 heads with RMSNorm + RoPE (R = 96) on Q in the kernel and
    each segment's own RoPE positions: bit-identical to the two-pass path, and sampled rows (the
    first and last query tile of every segment plus random rows) against the oracle composition."""
    import torch
    inp = gen.generate_qnorm([19394, 38000, 104000], 56, 96, seed=1008, name="qnorm_varlen_161394_h56")
    say("case attn_fwd_qnorm varlen pack")
    (o1, l1), (o2, l2), k_bits = _fused_and_two_pass(inp, gpu)
    assert np.array_equal(o1, o2) and np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    del o2, l2
    # the launch the benchmark times (the device's plan: 24 tail tiles x 8 ranges)
    import long_sequence_video_amd as lsv
    units = lsv.lsv_device_peak(0)[1]
    (o4, l4), (o5, l5), _ = _fused_and_two_pass(inp, gpu, units=units)
    assert np.array_equal(o4, o5) and np.array_equal(l4.view(np.uint32), l5.view(np.uint32))
    del o5, l5
    rows = sample_rows(inp, 24, seed=8)
    qref, _ = _oracle_rows(inp.q[rows], inp.q_weight, inp.cos[rows], inp.sin[rows], inp.eps)
    q_bits = np.zeros_like(inp.q)
    q_bits[rows] = gen.f64_to_bf16_bits(qref)
    comp = gen.Inputs(inp.name, q_bits, k_bits, inp.v, inp.cu_seqlens, inp.scale)
    compare(comp, o1, l1, rows=rows, label="qnorm varlen pack")
    from tests.gpu_common import whole_tile_rows
    whole, _, _ = whole_tile_rows(inp, units)
    cut = np.flatnonzero(~whole.all(axis=1))
    if len(cut):
        qref, _ = _oracle_rows(inp.q[cut], inp.q_weight, inp.cos[cut], inp.sin[cut], inp.eps)
        q_bits[cut] = gen.f64_to_bf16_bits(qref)
        comp = gen.Inputs(inp.name, q_bits, k_bits, inp.v, inp.cu_seqlens, inp.scale)
        compare(comp, o4, l4, rows=np.union1d(cut, rows), label="qnorm tail varlen pack")
    torch.cuda.empty_cache()
