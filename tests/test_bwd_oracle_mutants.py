"""Plant plausible mistakes in the attention-backward oracle (on the CPU); a pin must catch each."""

import numpy as np
import pytest

import oracle.attention_bwd as ob
from tests import test_bwd_oracle as pins

PIN_TESTS = [pins.test_b1_autograd, pins.test_b3_invariants, pins.test_b4_identical_keys]

MUTANTS = ["no_delta", "delta_sign", "dq_no_scale", "dk_no_scale", "dv_uses_dS", "dk_uses_p", "transpose_p",
           "dq_uses_v"]


def _make(mistake):
    """Replacements for the oracle's three steps (statistics, dQ rows, dK/dV rows), each with the
    planted mistake where it belongs and the plain arithmetic elsewhere."""
    real_stats = ob._stats

    def stats(hd, r0, r1, sigma, keep_o):
        real_stats(hd, r0, r1, sigma, keep_o)
        if mistake == "no_delta":
            hd.dvec[r0:r1] = 0.0
        if mistake == "delta_sign":
            hd.dvec[r0:r1] = -hd.dvec[r0:r1]

    def dq(hd, idx, sigma):
        p = np.exp((hd.qs[idx] @ hd.ks.T) * sigma - hd.lse[idx, None])
        ds = p * (hd.dos[idx] @ hd.vs.T - hd.dvec[idx, None])
        return (1.0 if mistake == "dq_no_scale" else sigma) * (ds @ (hd.vs if mistake == "dq_uses_v" else hd.ks))

    def dkdv(hd, idx, sigma):
        pt = np.exp((hd.ks[idx] @ hd.qs.T) * sigma - hd.lse[None, :])
        if mistake == "transpose_p":
            pt = np.exp((hd.qs[idx] @ hd.ks.T) * sigma - hd.lse[idx, None])
        dst = pt * (hd.vs[idx] @ hd.dos.T - hd.dvec[None, :])
        dv = (dst if mistake == "dv_uses_dS" else pt) @ hd.dos
        dk = (1.0 if mistake == "dk_no_scale" else sigma) * ((pt if mistake == "dk_uses_p" else dst) @ hd.qs)
        return dk, dv
    return stats, dq, dkdv


@pytest.mark.parametrize("mistake", MUTANTS)
def test_pins_catch_mutant(mistake, monkeypatch):
    stats, dq, dkdv = _make(mistake)
    monkeypatch.setattr(ob, "_stats", stats)
    monkeypatch.setattr(ob, "_dq", dq)
    monkeypatch.setattr(ob, "_dkdv", dkdv)
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {mistake!r}"


def test_unmutated_steps_pass_the_pins(monkeypatch):
    """The replacement steps with no mistake are the oracle itself: every pin passes."""
    stats, dq, dkdv = _make("none")
    monkeypatch.setattr(ob, "_stats", stats)
    monkeypatch.setattr(ob, "_dq", dq)
    monkeypatch.setattr(ob, "_dkdv", dkdv)
    for t in PIN_TESTS:
        t()
