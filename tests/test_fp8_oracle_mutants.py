"""Plant plausible mistakes in the FP8 oracle (on the CPU); a pin must catch each."""

import numpy as np
import pytest

import oracle.attention_fp8 as of
from tests import test_fp8_oracle as pins

PIN_TESTS = [pins.test_f1_format_definition, pins.test_f3_matches_bf16_oracle]
REAL_DECODE = of.e4m3_bits_to_f64


def _decoder(mistake):
    def dec(bits):
        b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
        sign = np.where(b & 0x80, -1.0, 1.0)
        e = (b >> 3) & 0xF
        m = b & 0x7
        bias = 8 if mistake == "bias8" else 7
        sub = (1.0 + m / 8.0) * 2.0 ** -6 if mistake == "subnormal_implicit_one" else m * 2.0 ** -9
        val = np.where(e == 0, sub, (1.0 + m / 8.0) * 2.0 ** (e - bias))
        if mistake == "mantissa_16ths":
            val = np.where(e == 0, sub, (1.0 + m / 16.0) * 2.0 ** (e - bias))
        val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
        return (1.0 if mistake == "no_sign" else sign) * val
    return dec


def _attention(mistake):
    real = of.attention_fp8_fp64

    def att(q8, k8, v8, dq, dk, dv, cu, scale, *, rows=None):
        if mistake == "ignore_dv":
            dv = 1.0
        if mistake == "dq_squared":
            dk = dq
        return real(q8, k8, v8, dq, dk, dv, cu, scale, rows=rows)
    return att


@pytest.mark.parametrize("mistake", ["bias8", "subnormal_implicit_one", "mantissa_16ths", "no_sign"])
def test_pins_catch_decoder_mutant(mistake, monkeypatch):
    monkeypatch.setattr(of, "e4m3_bits_to_f64", _decoder(mistake))
    monkeypatch.setattr(pins, "e4m3_bits_to_f64", _decoder(mistake))
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, mistake


@pytest.mark.parametrize("mistake", ["ignore_dv", "dq_squared"])
def test_pins_catch_descale_mutant(mistake, monkeypatch):
    monkeypatch.setattr(pins, "attention_fp8_fp64", _attention(mistake))
    with pytest.raises(AssertionError):
        pins.test_f3_matches_bf16_oracle()
