"""Pins of the fp64 attention-backward oracle against facts that do not come from it.

* B1 autograd: torch float64 autograd through a plain softmax attention (per segment)
  with grad_output dO gives the same dQ, dK, dV.
* B2 finite differences: central differences of the *forward* oracle's
  ``L = sum(dO * O)`` match single entries of dQ, dK, dV.
* B3 invariants: per (segment, head) ``sum_j dK_j = 0`` (softmax is invariant to a common
  shift of the keys) and ``sum_j dV_j = sum_i dO_i`` (each row of P sums to 1).
* B4 identical keys: P is uniform, so dQ = 0 and every dV_j = mean_i dO_i.
* B5 segment isolation: changing one segment's data leaves the others' gradients identical.
* B6 row subsets equal the full result; empty and bad inputs.
"""

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen
from oracle import attention_bwd_fp64, attention_fp64, bf16_bits_to_f64


def _case(seqlens, heads, d=128, seed=3):
    inp = gen.generate(seqlens, heads, d, seed=seed, name="bwd")
    do = gen.normal_bf16(inp.q.size, seed, 9).reshape(inp.q.shape)
    return inp, do


def test_b1_autograd():
    import torch
    inp, do = _case([37, 0, 20], 2, d=128)
    res = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    sigma = float(np.float64(np.float32(inp.scale)))
    q = torch.tensor(bf16_bits_to_f64(inp.q), requires_grad=True)
    k = torch.tensor(bf16_bits_to_f64(inp.k), requires_grad=True)
    v = torch.tensor(bf16_bits_to_f64(inp.v), requires_grad=True)
    outs = []
    cu = inp.cu_seqlens
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            qs, ks, vs = (t[a:b].transpose(0, 1) for t in (q, k, v))   # [H, L, D]
            p = torch.softmax(sigma * qs @ ks.transpose(1, 2), dim=-1)
            outs.append((p @ vs).transpose(0, 1))
    out = torch.cat(outs)
    out.backward(torch.tensor(bf16_bits_to_f64(do)))
    np.testing.assert_allclose(res["dq"], q.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(res["dk"], k.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(res["dv"], v.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_b2_finite_differences():
    """The forward oracle is differentiated numerically: one bf16 input entry moves to its
    two neighbouring bf16 values (exact inputs on both sides), the forward oracle evaluates
    L at both, and the divided difference must match the backward oracle's entry."""
    inp, do = _case([12], 1, d=128, seed=11)
    res = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    dof = bf16_bits_to_f64(do)

    def loss(q, k, v):
        out, _, _ = attention_fp64(q, k, v, inp.cu_seqlens, inp.scale)
        return float(np.sum(out * dof))

    checked = 0
    for name, grad in (("q", res["dq"]), ("k", res["dk"]), ("v", res["dv"])):
        for (t, d) in ((3, 5), (7, 100), (11, 64)):
            x = getattr(inp, name)
            # symmetric bf16 neighbours of x[t, 0, d]: x - ulp and x + ulp (exact values)
            base = int(x[t, 0, d])
            hi, lo = x.copy(), x.copy()
            hi[t, 0, d] = base + 1 if not (base & 0x8000) else base - 1   # one ulp away from zero
            lo[t, 0, d] = base - 1 if not (base & 0x8000) else base + 1   # one ulp towards zero
            xh = bf16_bits_to_f64(hi[t, 0, d])
            xl = bf16_bits_to_f64(lo[t, 0, d])
            args_h = {n: getattr(inp, n) for n in "qkv"}
            args_l = dict(args_h)
            args_h[name], args_l[name] = hi, lo
            fd = (loss(args_h["q"], args_h["k"], args_h["v"]) - loss(args_l["q"], args_l["k"], args_l["v"])) / (xh - xl)
            g = grad[t, 0, d]
            assert abs(fd - g) <= 2e-3 * (abs(g) + 1e-3), (name, t, d, fd, g)
            checked += 1
    assert checked == 9


def test_b3_invariants():
    inp, do = _case([300, 77], 3, seed=12)
    res = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    dof = bf16_bits_to_f64(do)
    cu = inp.cu_seqlens
    for a, b in zip(cu[:-1], cu[1:]):
        sdk = res["dk"][a:b].sum(axis=0)
        assert np.abs(sdk).max() < 1e-10 * (1 + np.abs(res["dk"][a:b]).sum(axis=0).max())
        np.testing.assert_allclose(res["dv"][a:b].sum(axis=0), dof[a:b].sum(axis=0), rtol=1e-11, atol=1e-11)


def test_b4_identical_keys():
    inp, do = _case([50], 2, seed=13)
    inp.k[:] = inp.k[7]
    res = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    dof = bf16_bits_to_f64(do)
    assert np.abs(res["dq"]).max() < 1e-12
    np.testing.assert_allclose(res["dv"], np.broadcast_to(dof.mean(axis=0), res["dv"].shape), rtol=1e-12,
                               atol=1e-13)


def test_b5_segment_isolation():
    inp, do = _case([40, 60], 2, seed=14)
    r1 = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    inp.q[40:] = inp.q[40:][::-1].copy()
    inp.v[40:] = 0x3F80  # 1.0
    do2 = do.copy()
    do2[40:] = 0xBF80
    r2 = attention_bwd_fp64(inp.q, inp.k, inp.v, do2, inp.cu_seqlens, inp.scale)
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(r1[key][:40], r2[key][:40])
        assert not np.array_equal(r1[key][40:], r2[key][40:])


def test_b6_row_subsets_and_edges():
    inp, do = _case([33, 0, 70], 2, seed=15)
    full = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale)
    qr = np.array([0, 32, 33, 90, 102])
    kr = np.array([5, 40, 41])
    sub = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale, q_rows=qr, k_rows=kr)
    np.testing.assert_allclose(sub["dq"], full["dq"][qr], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sub["dk"], full["dk"][kr], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(sub["dv"], full["dv"][kr], rtol=1e-13, atol=1e-15)
    # a single-key segment: P = 1, dS = 0: dQ = dK = 0 and dV = dO
    one, do1 = _case([1], 2, seed=16)
    r = attention_bwd_fp64(one.q, one.k, one.v, do1, one.cu_seqlens, one.scale)
    assert np.abs(r["dq"]).max() < 1e-15 and np.abs(r["dk"]).max() < 1e-15
    np.testing.assert_array_equal(r["dv"], bf16_bits_to_f64(do1))
    with pytest.raises(ValueError):
        attention_bwd_fp64(inp.q, inp.k, inp.v, do[:5], inp.cu_seqlens, inp.scale)
    with pytest.raises(ValueError):
        attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale, q_rows=np.array([33 + 0, 500]))


def test_b7_forward_outputs_and_thread_count():
    """``return_forward`` gives the forward oracle's O and LSE on every row of the segments it
    touched, zeros elsewhere; the gradients do not depend on the thread count or on how rows
    are split into blocks (a long segment is spread over threads block by block)."""
    import oracle.attention_bwd as ob
    inp, do = _case([300, 0, 45], 2, seed=21)
    inp = gen.Inputs("b7", inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale)
    q_rows = np.array([0, 7, 299, 300, 344])
    k_rows = np.array([3, 150, 301])
    one = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale, q_rows=q_rows, k_rows=k_rows,
                             workers=1, return_forward=True)
    o, l, rows = attention_fp64(inp.q, inp.k, inp.v, inp.cu_seqlens, inp.scale)
    np.testing.assert_allclose(one["o"][rows], o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(one["lse"][:, rows], l, rtol=1e-12, atol=1e-14)
    old = ob._ELEMS
    try:
        ob._ELEMS = 300 * 8          # blocks of 8 rows: many blocks, many threads
        many = attention_bwd_fp64(inp.q, inp.k, inp.v, do, inp.cu_seqlens, inp.scale, q_rows=q_rows,
                                  k_rows=k_rows, workers=4)
    finally:
        ob._ELEMS = old
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(many[name], one[name], rtol=1e-12, atol=1e-14)
