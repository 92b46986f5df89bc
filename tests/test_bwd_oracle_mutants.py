"""Plant plausible mistakes in the attention-backward oracle (on the CPU); a pin must catch each."""

import numpy as np
import pytest

import oracle.attention_bwd as ob
from tests import test_bwd_oracle as pins

PIN_TESTS = [pins.test_b1_autograd, pins.test_b3_invariants, pins.test_b4_identical_keys]

MUTANTS = ["no_delta", "delta_sign", "dq_no_scale", "dk_no_scale", "dv_uses_dS", "dk_uses_p", "transpose_p",
           "dq_uses_v"]


def _make(mistake):
    real_stats = ob._stats

    def one(q, k, v, do, a, b, h, q_rows, k_rows, sigma):
        qs = ob.bf16_bits_to_f64(q[a:b, h, :])
        ks = ob.bf16_bits_to_f64(k[a:b, h, :])
        vs = ob.bf16_bits_to_f64(v[a:b, h, :])
        dos = ob.bf16_bits_to_f64(do[a:b, h, :])
        lse, dvec = real_stats(qs, ks, vs, dos, sigma)
        if mistake == "no_delta":
            dvec = np.zeros_like(dvec)
        if mistake == "delta_sign":
            dvec = -dvec
        iq = q_rows - a
        p = np.exp((qs[iq] @ ks.T) * sigma - lse[iq, None])
        ds = p * (dos[iq] @ vs.T - dvec[iq, None])
        dq = (1.0 if mistake == "dq_no_scale" else sigma) * (ds @ (vs if mistake == "dq_uses_v" else ks))
        ik = k_rows - a
        pt = np.exp((ks[ik] @ qs.T) * sigma - lse[None, :])
        if mistake == "transpose_p":
            pt = np.exp((qs[ik] @ ks.T) * sigma - lse[ik, None])
        dst = pt * (vs[ik] @ dos.T - dvec[None, :])
        dv = (dst if mistake == "dv_uses_dS" else pt) @ dos
        dk = (1.0 if mistake == "dk_no_scale" else sigma) * ((pt if mistake == "dk_uses_p" else dst) @ qs)
        return dq, dk, dv
    return one


@pytest.mark.parametrize("mistake", MUTANTS)
def test_pins_catch_mutant(mistake, monkeypatch):
    monkeypatch.setattr(ob, "_one", _make(mistake))
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {mistake!r}"
