"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Every mutant replaces the oracle's per-head kernel with a copy carrying one
mistake; the pins of ``test_oracle.py`` run against it and at least one must fail.
"""

import numpy as np
import pytest

import oracle.attention as oa
from tests import test_oracle as pins

PIN_TESTS = [
    pins.test_identical_keys_give_mean_of_values,
    pins.test_dominant_logit_selects_its_value_row,
    pins.test_brute_force_tiny,
    pins.test_segments_are_isolated,
    pins.test_tiny_scale_limit,
    pins.test_library_cross_check,
    pins.test_single_key_segment,
]


def _make(mistake):
    def head_rows(q, k, v, a, b, h, rows, sigma):
        H = q.shape[1]
        ka, kb = (0, b) if mistake == "segment_leak" else (a, b)
        hk = (h + 1) % H if mistake == "head_mixup" else h
        ks = oa.bf16_bits_to_f64(k[ka:kb, hk, :])
        vs = oa.bf16_bits_to_f64((k if mistake == "k_for_v" else v)[ka:kb, h, :])
        qb = oa.bf16_bits_to_f64(q[rows, h, :])
        s = 1.0 if mistake == "no_scale" else (sigma * sigma if mistake == "scale_twice" else sigma)
        z = (qb @ ks.T) * s
        if mistake == "off_by_one_key" and z.shape[1] > 1:
            z, vs = z[:, :-1], vs[:-1]
        m = z.max(axis=1)
        e = np.exp(z - m[:, None]) if mistake != "sign" else np.exp(m[:, None] - z)
        l = e.sum(axis=1)
        out = (e @ vs) / (l[:, None] if mistake != "no_normalise" else 1.0)
        if mistake == "lse_log2":
            lse = m + np.log2(l)
        elif mistake == "lse_no_max":
            lse = np.log(l)
        else:
            lse = m + np.log(l)
        return out, lse
    return head_rows


MUTANTS = ["segment_leak", "head_mixup", "k_for_v", "no_scale", "scale_twice", "off_by_one_key",
           "sign", "no_normalise", "lse_log2", "lse_no_max"]


@pytest.mark.parametrize("mistake", MUTANTS)
def test_pins_catch_mutant(mistake, monkeypatch):
    monkeypatch.setattr(oa, "_head_rows", _make(mistake))
    caught = []
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError):
            caught.append(t.__name__)
    assert caught, f"no pin caught the '{mistake}' mutant"


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(oa, "_head_rows", _make("none"))
    for t in PIN_TESTS:
        t()
