"""Pins of the e4m3 decoder and the fp64 FP8-attention oracle.

* F1 the OCP e4m3 format by its definition: hand-listed codes (zero, the smallest
  subnormal, the largest subnormal, the smallest normal, one, the largest finite value,
  NaN, sign) and every code's value rebuilt from its fields with pure-Python arithmetic.
* F2 the input quantiser: round trip of every finite code, round-to-nearest-even ties,
  saturation.
* F3 the FP8 oracle equals the (pinned) BF16 oracle on the same values: every e4m3 value is
  a bf16 value, so with unit descales the two definitions coincide; power-of-two descales
  fold into the scale (dq, dk) and scale the output (dv) exactly.
"""

import math

import numpy as np

from long_sequence_video_amd import inputs as gen
from oracle import attention_fp64, attention_fp8_fp64, e4m3_bits_to_f64


def test_f1_format_definition():
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5, 0x45: 3.25}
    for code, val in known.items():
        assert e4m3_bits_to_f64(np.uint8(code)) == val, hex(code)
    assert math.isnan(e4m3_bits_to_f64(np.uint8(0x7F))) and math.isnan(e4m3_bits_to_f64(np.uint8(0xFF)))
    codes = np.arange(256, dtype=np.uint8)
    got = e4m3_bits_to_f64(codes)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert got[c] == (-v if s else v), hex(c)


def test_f2_quantiser():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3_bits_to_f64(finite)
    back = gen.f64_to_e4m3_bits(vals)
    assert np.array_equal(e4m3_bits_to_f64(back), vals)  # -0 and +0 compare equal
    ties = np.array([2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 248.0, 17.0])
    assert list(e4m3_bits_to_f64(gen.f64_to_e4m3_bits(ties))) == [0.0, 2 * 2.0 ** -9, 1.0, 1.25, 256.0, 16.0]
    assert list(e4m3_bits_to_f64(gen.f64_to_e4m3_bits([1000.0, -1e9, 449.0]))) == [448.0, -448.0, 448.0]


def _as_bf16_bits(b8):
    """e4m3 bytes -> the bf16 bit patterns of the same values (exact)."""
    return gen.f64_to_bf16_bits(e4m3_bits_to_f64(b8))


def test_f3_matches_bf16_oracle():
    inp = gen.generate([200, 0, 57], 3, seed=41, name="f3")
    f8 = gen.quantize_fp8(inp)
    q, k, v = (_as_bf16_bits(x) for x in (f8.q, f8.k, f8.v))
    assert np.array_equal(e4m3_bits_to_f64(f8.q), (q.astype(np.uint32) << 16).view(np.float32))
    o1, l1, _ = attention_fp8_fp64(f8.q, f8.k, f8.v, 1.0, 1.0, 1.0, f8.cu_seqlens, 0.125)
    o2, l2, _ = attention_fp64(q, k, v, f8.cu_seqlens, 0.125)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)
    # power-of-two descales: dq dk fold into the scale, dv scales the output
    o3, l3, _ = attention_fp8_fp64(f8.q, f8.k, f8.v, 0.5, 0.25, 4.0, f8.cu_seqlens, 0.125)
    o4, l4, _ = attention_fp64(q, k, v, f8.cu_seqlens, 0.125 * 0.5 * 0.25)
    np.testing.assert_allclose(o3, 4.0 * o4, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=1e-12, atol=1e-12)


def test_quantised_workload_shapes():
    inp = gen.generate([300], 2, seed=42, name="fq")
    f8 = gen.quantize_fp8(inp)
    assert f8.q.dtype == np.uint8 and f8.q.shape == inp.q.shape
    for key in ("q", "k", "v"):
        x = e4m3_bits_to_f64(getattr(f8, key)) * getattr(f8, "descale_" + key)
        ref = (getattr(inp, key).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.abs(x).max() <= 448 * getattr(f8, "descale_" + key) * (1 + 1e-7)
        assert np.abs(x - ref).max() <= 0.0625 * np.abs(ref).max()   # e4m3 half-ulp bound, relative to amax
