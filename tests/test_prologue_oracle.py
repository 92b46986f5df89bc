"""Pins of the fp64 QKV-prologue oracle against facts that do not come from the oracle itself.

* PR1 library RMSNorm: with no rotation the result equals ``torch.nn.functional.rms_norm``
  in float64 (an independent routine) with the same weight and eps.
* PR2 complex rotation: with true RoPE tables (channels i and i + R/2 share one angle),
  the rotated channels equal the complex product ``(y_i + j y_{i+R/2}) e^{j theta_i}``
  computed with torch complex128 on the library-normalised rows.
* PR3 rotation preserves each pair's norm: ``out_i^2 + out_{i+R/2}^2 = y_i^2 + y_{i+R/2}^2``.
* PR4 relative position: for RoPE tables ``<R_m a, R_n b>`` over the rotated channels
  depends only on ``m - n``.
* PR5 RMS closed form: unit weight, no rotation: ``mean(out^2) = ms / (ms + eps)``.
* PR6 scale invariance: with eps = 0, scaling a row by 2 (exact in bf16) leaves the
  output unchanged.
* PR7 tiny brute force: pure-Python ``math.fsum`` / ``math.sqrt`` loops on a few rows.
* PR8 the page's shapes: stacked output planes and the V copy (golden fixture).
"""

import json
import math
import os

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import bf16_bits_to_f64, norm_rope_rows_fp64, qkv_prologue_fp64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qkv_prologue_shape_pin.json")


def _rows(n, d=128, seed=5, tensor=0):
    return gen.normal_bf16(n * d, seed, tensor).reshape(n, d)


def _torch_rms(x_bits, w_bits, eps):
    import torch
    x = torch.from_numpy(bf16_bits_to_f64(x_bits))
    w = torch.from_numpy(bf16_bits_to_f64(w_bits))
    e = float(np.float64(np.float32(eps)))
    return torch.nn.functional.rms_norm(x, (x.shape[-1],), weight=w, eps=e).numpy()


def test_pr1_library_rmsnorm_without_rotation():
    x = _rows(64)
    w = gen.normal_bf16(128, 9, 4)
    empty = np.zeros((64, 0), dtype=np.uint16)
    out, _ = norm_rope_rows_fp64(x, w, empty, empty, 1e-5)
    np.testing.assert_allclose(out, _torch_rms(x, w, 1e-5), rtol=1e-13, atol=1e-13)
    # with R = 96 the unrotated channels are the same normalised values
    cos, sin = gen.rope_tables(64, 96)
    out96, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
    np.testing.assert_allclose(out96[:, 96:], _torch_rms(x, w, 1e-5)[:, 96:], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rd", [96, 128, 32])
def test_pr2_complex_rotation(rd):
    import torch
    n = 40
    x = _rows(n, seed=6)
    w = gen.normal_bf16(128, 10, 4)
    cos, sin = gen.rope_tables(n, rd, start=1000)
    out, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
    y = torch.from_numpy(_torch_rms(x, w, 1e-5))
    h = rd // 2
    c = torch.from_numpy(bf16_bits_to_f64(cos[:, :h]))
    s = torch.from_numpy(bf16_bits_to_f64(sin[:, :h]))
    z = torch.complex(y[:, :h], y[:, h:rd]) * torch.complex(c, s)
    np.testing.assert_allclose(out[:, :h], z.real.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[:, h:rd], z.imag.numpy(), rtol=1e-12, atol=1e-12)


def test_pr3_pair_norm_preserved():
    n = 50
    x = _rows(n, seed=7)
    w = gen.normal_bf16(128, 11, 4)
    # tables that are exact rotations in bf16: quarter and half turns
    for cval, sval in ((0.0, 1.0), (-1.0, 0.0), (0.0, -1.0)):
        cos = gen.f64_to_bf16_bits(np.full((n, 96), cval))
        sin = gen.f64_to_bf16_bits(np.full((n, 96), sval))
        out, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
        y = _torch_rms(x, w, 1e-5)
        np.testing.assert_allclose(out[:, :48] ** 2 + out[:, 48:96] ** 2, y[:, :48] ** 2 + y[:, 48:96] ** 2,
                                   rtol=1e-12, atol=1e-14)
    # bf16-rounded RoPE tables are rotations up to the table rounding (|c^2 + s^2 - 1| < 2^-7)
    cos, sin = gen.rope_tables(n, 96, start=7)
    out, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
    c = bf16_bits_to_f64(cos[:, :48])
    s = bf16_bits_to_f64(sin[:, :48])
    y = _torch_rms(x, w, 1e-5)
    np.testing.assert_allclose(out[:, :48] ** 2 + out[:, 48:96] ** 2,
                               (c * c + s * s) * (y[:, :48] ** 2 + y[:, 48:96] ** 2), rtol=1e-12, atol=1e-14)


def test_pr4_relative_position():
    """An exact identity needs tables that are exact rotations in bf16: every angle here is
    a multiple of a quarter turn."""
    d, rd = 128, 96
    a = _rows(1, seed=8)
    b = _rows(1, seed=8, tensor=1)
    w = gen.normal_bf16(d, 12, 4)

    def rot(x, p):
        # frequency of pair i: (i % 4) quarter turns per position step
        ang = np.array([(p * (i % 4)) % 4 for i in range(rd // 2)], dtype=np.float64) * (math.pi / 2)
        ang = np.concatenate([ang, ang])
        cos = gen.f64_to_bf16_bits(np.round(np.cos(ang))[None])
        sin = gen.f64_to_bf16_bits(np.round(np.sin(ang))[None])
        out, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
        return out[0, :rd]

    d1 = rot(a, 5) @ rot(b, 2)
    d2 = rot(a, 13) @ rot(b, 10)
    d3 = rot(a, 6) @ rot(b, 2)
    assert abs(d1 - d2) < 1e-12 * (1 + abs(d1))
    assert abs(d1 - d3) > 1e-3  # a different offset gives a different product


def test_pr5_rms_closed_form():
    x = _rows(32, seed=13)
    one = gen.f64_to_bf16_bits(np.ones(128))
    empty = np.zeros((32, 0), dtype=np.uint16)
    eps = 0.25  # exact in fp32; large enough to matter
    out, _ = norm_rope_rows_fp64(x, one, empty, empty, eps)
    xf = bf16_bits_to_f64(x)
    ms = np.mean(xf * xf, axis=1)
    np.testing.assert_allclose(np.mean(out * out, axis=1), ms / (ms + 0.25), rtol=1e-13)


def test_pr6_scale_invariance_without_eps():
    x = _rows(16, seed=14)
    x2 = gen.f64_to_bf16_bits(2.0 * bf16_bits_to_f64(x))
    w = gen.normal_bf16(128, 15, 4)
    cos, sin = gen.rope_tables(16, 96)
    o1, _ = norm_rope_rows_fp64(x, w, cos, sin, 0.0)
    o2, _ = norm_rope_rows_fp64(x2, w, cos, sin, 0.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)


def test_pr7_brute_force_rows():
    x = _rows(3, seed=16)
    w = gen.normal_bf16(128, 17, 4)
    cos = gen.normal_bf16(3 * 96, 18, 6).reshape(3, 96)
    sin = gen.normal_bf16(3 * 96, 18, 7).reshape(3, 96)
    out, _ = norm_rope_rows_fp64(x, w, cos, sin, 1e-5)
    eps = float(np.float32(1e-5))
    for r in range(3):
        xs = [float(t) for t in bf16_bits_to_f64(x[r])]
        ws = [float(t) for t in bf16_bits_to_f64(w)]
        cs = [float(t) for t in bf16_bits_to_f64(cos[r])]
        ss = [float(t) for t in bf16_bits_to_f64(sin[r])]
        inv = 1.0 / math.sqrt(math.fsum(t * t for t in xs) / 128 + eps)
        y = [xs[i] * inv * ws[i] for i in range(128)]
        for i in range(128):
            if i < 48:
                ref = y[i] * cs[i] - y[i + 48] * ss[i]
            elif i < 96:
                ref = y[i] * cs[i] + y[i - 48] * ss[i]
            else:
                ref = y[i]
            assert abs(out[r, i] - ref) <= 1e-12 * (1 + abs(ref))


def test_pr8_page_shapes_and_v_copy():
    pin = json.load(open(GOLDEN))
    b, s, h, d, rd = 2, 7, 3, 128, pin["rotary_dim"]
    inp = gen.generate_prologue(b, s, h, d, rd, seed=19, tables="normal")
    res = qkv_prologue_fp64(inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin, inp.eps)
    assert res["q"].shape == (b * s, h, d) and res["k"].shape == (b * s, h, d)
    assert np.array_equal(res["v"], inp.v.reshape(b * s, h, d))
    # per-position tables: token b*S + p uses row p
    one = qkv_prologue_fp64(inp.q[1:2], inp.k[1:2], inp.v[1:2], inp.q_weight, inp.k_weight, inp.cos, inp.sin,
                            inp.eps)
    np.testing.assert_array_equal(one["q"], res["q"][s:])
    # the page's int32-plane shape: each plane has more than 2^30 elements
    B, S, H, D, R = pin["int32_plane_shape"]
    assert B * S * H * D == pin["plane_elements"] and 2 * B * S * H * D > 2 ** 31 and R == rd
    assert pin["out_planes"] == 3


def test_token_subset_matches_full():
    inp = gen.generate_prologue(1, 20, 2, seed=20)
    full = qkv_prologue_fp64(inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin)
    sub = qkv_prologue_fp64(inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin,
                            tokens=np.array([3, 17]))
    np.testing.assert_array_equal(sub["q"], full["q"][[3, 17]])
    np.testing.assert_array_equal(sub["k_mag"], full["k_mag"][[3, 17]])


def test_bad_arguments():
    x = _rows(2)
    w = gen.normal_bf16(128, 1, 4)
    with pytest.raises(ValueError):
        norm_rope_rows_fp64(x, w, np.zeros((2, 95), np.uint16), np.zeros((2, 95), np.uint16), 1e-5)
    with pytest.raises(ValueError):
        norm_rope_rows_fp64(x, w[:64], np.zeros((2, 0), np.uint16), np.zeros((2, 0), np.uint16), 1e-5)
    inp = gen.generate_prologue(1, 4, 2, seed=1)
    with pytest.raises(ValueError):
        qkv_prologue_fp64(inp.q, inp.k[:, :3], inp.v, inp.q_weight, inp.k_weight, inp.cos, inp.sin)
    with pytest.raises(ValueError):
        qkv_prologue_fp64(inp.q, inp.k, inp.v, inp.q_weight, inp.k_weight, inp.cos[:3], inp.sin[:3])
