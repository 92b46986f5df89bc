"""Plant plausible mistakes in the QKV-prologue oracle (on the CPU); a pin must catch each."""

import numpy as np
import pytest

import oracle.prologue as op
from oracle.attention import bf16_bits_to_f64, f32_to_f64
from tests import test_prologue_oracle as pins

PIN_TESTS = [
    pins.test_pr1_library_rmsnorm_without_rotation,
    lambda: pins.test_pr2_complex_rotation(96),
    pins.test_pr3_pair_norm_preserved,
    pins.test_pr4_relative_position,
    pins.test_pr5_rms_closed_form,
    pins.test_pr6_scale_invariance_without_eps,
]

MUTANTS = ["sum_not_mean", "eps_outside_sqrt", "no_weight", "sign_swapped", "partner_shift",
           "interleaved_pairs", "rotate_all", "weight_before_norm_sq"]


def _make(mistake):
    def rows(x_bits, w_bits, cos_bits, sin_bits, eps):
        x = bf16_bits_to_f64(x_bits)
        w = bf16_bits_to_f64(w_bits)
        c = bf16_bits_to_f64(cos_bits)
        s = bf16_bits_to_f64(sin_bits)
        r = c.shape[1]
        e = f32_to_f64(eps)
        if mistake == "weight_before_norm_sq":
            xw = x * w[None, :]
            inv = 1.0 / np.sqrt(np.mean(xw * xw, axis=1) + e)
            y = xw * inv[:, None]
        else:
            ms = np.sum(x * x, axis=1) if mistake == "sum_not_mean" else np.mean(x * x, axis=1)
            inv = 1.0 / np.sqrt(ms) + e if mistake == "eps_outside_sqrt" else 1.0 / np.sqrt(ms + e)
            y = x * inv[:, None] * (1.0 if mistake == "no_weight" else w[None, :])
        out = y.copy()
        h = r // 2
        if h:
            if mistake == "interleaved_pairs":
                a, b = y[:, 0:r:2], y[:, 1:r:2]
                out[:, 0:r:2] = a * c[:, 0:r:2] - b * s[:, 0:r:2]
                out[:, 1:r:2] = b * c[:, 1:r:2] + a * s[:, 1:r:2]
            else:
                lo, hi = y[:, :h], y[:, h:r]
                if mistake == "partner_shift":
                    hi = np.roll(hi, 1, axis=1)
                sg = -1.0 if mistake == "sign_swapped" else 1.0
                out[:, :h] = lo * c[:, :h] - sg * hi * s[:, :h]
                out[:, h:r] = y[:, h:r] * c[:, h:r] + sg * lo * s[:, h:r]
            if mistake == "rotate_all" and r < y.shape[1]:
                out[:, r:] = -y[:, r:]
        return out, np.abs(out)
    return rows


@pytest.mark.parametrize("mistake", MUTANTS)
def test_pins_catch_mutant(mistake, monkeypatch):
    monkeypatch.setattr(op, "norm_rope_rows_fp64", _make(mistake))
    monkeypatch.setattr(pins, "norm_rope_rows_fp64", _make(mistake))
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {mistake!r}"
