"""GPU parity of the HIP QKV prologue against the fp64 oracle, through the C ABI.

Bar (the kernel computes in fp32 and rounds once to bf16): every element of rotated Q/K is
within one bf16 ulp of the exact value plus a cancellation allowance (``2^-7 |ref| +
2^-16 * sum of |terms|``); at least 99.9% of the elements equal the exact value rounded to
nearest even; the rel-L2 distance to that rounded value is below the page's 1e-4; V is
copied bit for bit. Small shapes are checked on every element, the full-size shapes (the
161,394-token pack and the page's 4 x 40,000 x 56 batch whose V plane starts past 2^31
elements) on sampled tokens, with V compared in full on the device.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import bf16_bits_to_f64, qkv_prologue_fp64
from tests.gpu_common import from_dev, say, to_dev

pytestmark = pytest.mark.gpu


def run_prologue(inp, device, *, eps=None, keep_on_device=False):
    import torch
    import long_sequence_video_amd as lsv
    q, k, v = (to_dev(x, device) for x in (inp.q, inp.k, inp.v))
    qw, kw = to_dev(inp.q_weight, device), to_dev(inp.k_weight, device)
    rd = inp.rotary_dim
    cos = to_dev(inp.cos, device) if rd else None
    sin = to_dev(inp.sin, device) if rd else None
    out = lsv.qkv_prologue(q, k, v, qw, kw, cos, sin, eps=inp.eps if eps is None else eps)
    torch.cuda.synchronize(device)
    if keep_on_device:
        return out, v
    return from_dev(out)


def check(inp, out_bits, tokens=None, *, eps=None, label=""):
    """``out_bits``: uint16 [3, N, H, D] for the ``tokens`` (default: all)."""
    ref = qkv_prologue_fp64(inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin,
                            inp.eps if eps is None else eps, tokens=tokens)
    stats = {}
    for plane, name in ((0, "q"), (1, "k")):
        got_bits = out_bits[plane]
        got = bf16_bits_to_f64(got_bits)
        exact = ref[name]
        err = np.abs(got - exact)
        tol = 2.0 ** -7 * np.abs(exact) + 2.0 ** -16 * ref[name + "_mag"] + 1e-30
        rounded = gen.f64_to_bf16_bits(exact)
        same = float(np.mean(got_bits == rounded))
        rf = bf16_bits_to_f64(rounded)
        rel_l2 = float(np.linalg.norm(got - rf) / max(np.linalg.norm(rf), 1e-300))
        stats[name] = dict(max_err_over_tol=float((err / tol).max()), exact_rne=same, rel_l2=rel_l2)
        assert np.isfinite(got).all(), (label, name)
        assert (err <= tol).all(), (label, name, stats[name])
        assert same >= 0.999, (label, name, stats[name])
        assert rel_l2 < 1e-4, (label, name, stats[name])
    assert np.array_equal(out_bits[2], ref["v"]), (label, "v copy")
    say(f"[{label}] {stats}")
    return stats


@pytest.mark.parametrize("b,s,h,rd,tables", [
    (1, 1, 1, 96, "rope"),
    (2, 37, 3, 96, "rope"),
    (2, 37, 3, 96, "normal"),
    (1, 50, 5, 0, "normal"),
    (1, 50, 5, 128, "normal"),
    (3, 17, 2, 16, "rope"),
    (1, 33, 7, 32, "normal"),
    (1, 1000, 1, 96, "normal"),
])
def test_small_all_elements(gpu, b, s, h, rd, tables):
    inp = gen.generate_prologue(b, s, h, 128, rd, seed=100 + b + s + h + rd, tables=tables)
    say(f"case prologue b{b} s{s} h{h} rd{rd} {tables}")
    out = run_prologue(inp, gpu).reshape(3, b * s, h, 128)
    check(inp, out, label=f"b{b} s{s} h{h} rd{rd} {tables}")


@pytest.mark.parametrize("eps", [0.0, 0.25])
def test_eps_values(gpu, eps):
    inp = gen.generate_prologue(1, 64, 4, seed=7, tables="normal")
    say(f"case prologue eps {eps}")
    out = run_prologue(inp, gpu, eps=eps).reshape(3, 64, 4, 128)
    check(inp, out, eps=eps, label=f"eps {eps}")


def test_page_unit_shape_all_elements(gpu):
    inp = gen.make_prologue_config("prologue_s512_h56_randtab")
    say("case prologue_s512_h56_randtab")
    out = run_prologue(inp, gpu)
    assert out.shape == (3, 512, 56, 128)  # the page's output shape for B = 1
    check(inp, out, label="s512 h56 random tables")
    again = run_prologue(inp, gpu)
    assert np.array_equal(out, again)  # deterministic


def _sampled_tokens(n_tokens, seq_len, seed):
    rng = np.random.default_rng(seed)
    picks = [np.arange(min(64, n_tokens)), np.arange(max(0, n_tokens - 64), n_tokens),
             rng.integers(0, n_tokens, size=512)]
    if seq_len < n_tokens:  # batch boundaries
        edges = np.arange(seq_len, n_tokens, seq_len)
        picks += [edges, edges - 1]
    return np.unique(np.concatenate(picks))


def _check_large(inp, device, label):
    import torch
    out, v = run_prologue(inp, device, keep_on_device=True)
    b, s, h, d = inp.shape
    planes = out.view(3, b * s, h, d)
    say(f"[{label}] V plane equal on device")
    assert torch.equal(planes[2], v.view(b * s, h, d))
    tokens = _sampled_tokens(b * s, s, seed=b + s)
    idx = torch.from_numpy(tokens).to(device)
    sampled = from_dev(planes.index_select(1, idx))
    del out, v, planes
    torch.cuda.empty_cache()
    check(inp, sampled, tokens=tokens, label=label)


def test_bench_size_sampled(gpu):
    inp = gen.make_prologue_config("prologue_s161394_h56")
    say("case prologue_s161394_h56")
    _check_large(inp, gpu, "s161394 h56")


def test_page_int32_plane_shape_sampled(gpu):
    """The page's large-batch regression: B*S*H*D = 1.14688e9, so the V plane starts at
    2.29e9 elements (past 2^31)."""
    inp = gen.make_prologue_config("prologue_b4_s40000_h56")
    say("case prologue_b4_s40000_h56")
    _check_large(inp, gpu, "b4 s40000 h56")


def test_rejects_bad_shapes(gpu):
    import torch
    import long_sequence_video_amd as lsv
    x = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16, device=gpu)
    w = torch.zeros(128, dtype=torch.bfloat16, device=gpu)
    t = torch.zeros((4, 40), dtype=torch.bfloat16, device=gpu)
    with pytest.raises(lsv.LsvError) as e:
        lsv.qkv_prologue(x, x, x, w, w, t, t)
    assert e.value.status == lsv.LSV_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        lsv.qkv_prologue(x, x, x, w, w, t[:3], t[:3])
