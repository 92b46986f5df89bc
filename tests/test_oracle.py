"""Pins for the fp64 oracle, checked against what the pages and the mathematics fix.

Each test targets a different plausible mistake in the oracle: segment leakage,
a transposed operand, a missing or doubled scale, the LSE base, a dropped max
shift, a head mix-up. None of them re-derives the oracle's own expression.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention_fp64, bf16_bits_to_f64, f32_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (via float32, nearest even) as uint16 bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def rand_bits(rng, shape, scale=1.0):
    return f64_to_bf16_bits(rng.standard_normal(shape) * scale)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3F81, 0x7F7F], dtype=np.uint16)
    want = [1.0, -1.0, 2.0, 0.0, -0.0, 1.0 + 2.0 ** -7, (2 - 2.0 ** -7) * 2.0 ** 127]
    np.testing.assert_array_equal(bf16_bits_to_f64(bits), np.array(want))


def test_shape_pin_from_pages():
    """The varlen interface example printed on the FastVideo #2049 page."""
    pin = json.load(open(os.path.join(GOLDEN, "varlen_shape_pin.json")))
    rng = np.random.default_rng(0)
    q = rand_bits(rng, pin["q_shape"])
    out, lse, rows = attention_fp64(q, q.copy(), q.copy(), pin["cu_seqlens"], pin["softmax_scale"])
    assert list(out.shape) == pin["out_shape"]
    assert list(lse.shape) == pin["lse_shape"]
    assert f32_to_f64(pin["softmax_scale"]) == 0.125


def test_identical_keys_give_mean_of_values():
    """T1: all keys of a segment equal k0 -> O = mean(V), LSE = sigma q.k0 + ln L."""
    rng = np.random.default_rng(1)
    seqlens, H, D = [5, 11, 1], 3, 16
    T = sum(seqlens)
    q = rand_bits(rng, (T, H, D))
    v = rand_bits(rng, (T, H, D))
    k = np.empty_like(q)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    for a, b in zip(cu[:-1], cu[1:]):
        k[a:b] = rand_bits(rng, (1, H, D))  # one key vector per segment and head
    scale = 0.3
    out, lse, _ = attention_fp64(q, k, v, cu, scale)
    qf, kf, vf = (bf16_bits_to_f64(x) for x in (q, k, v))
    sigma = f32_to_f64(scale)
    for a, b in zip(cu[:-1], cu[1:]):
        L = b - a
        for h in range(H):
            np.testing.assert_allclose(out[a:b, h], np.broadcast_to(vf[a:b, h].mean(0), (L, D)),
                                       rtol=0, atol=1e-13)
            dots = np.array([math.fsum(qf[i, h] * kf[a, h]) for i in range(a, b)])
            np.testing.assert_allclose(lse[h, a:b], sigma * dots + math.log(L), rtol=0, atol=1e-12)


def test_dominant_logit_selects_its_value_row():
    """T2: key j* with a logit >= 60 above the rest -> O_i = V[j*] (to 1e-15)."""
    rng = np.random.default_rng(2)
    L, H, D = 40, 2, 128
    q = rand_bits(rng, (L, H, D))
    k = rand_bits(rng, (L, H, D), scale=0.05)
    v = rand_bits(rng, (L, H, D))
    i, jstar = 3, 29
    for h in range(H):
        k[jstar, h] = f64_to_bf16_bits(8.0 * bf16_bits_to_f64(q[i, h]))
    scale = 1.0 / math.sqrt(D)
    out, lse, _ = attention_fp64(q, k, v, [0, L], scale)
    qf, kf, vf = (bf16_bits_to_f64(x) for x in (q, k, v))
    sigma = f32_to_f64(scale)
    for h in range(H):
        z = np.array([sigma * math.fsum(qf[i, h] * kf[j, h]) for j in range(L)])
        gap = z[jstar] - np.max(np.delete(z, jstar))
        assert gap > 60
        np.testing.assert_allclose(out[i, h], vf[jstar, h], rtol=1e-15, atol=0)
        assert abs(lse[h, i] - z[jstar]) < 1e-12


def test_joint_key_value_permutation_is_invariant():
    """T3: permuting K and V rows together inside a segment changes nothing."""
    rng = np.random.default_rng(3)
    seqlens, H, D = [64, 37], 2, 128
    T = sum(seqlens)
    q, k, v = (rand_bits(rng, (T, H, D)) for _ in range(3))
    cu = np.array([0, 64, 101])
    perm = np.concatenate([rng.permutation(64), 64 + rng.permutation(37)])
    o1, l1, _ = attention_fp64(q, k, v, cu, 0.0884)
    o2, l2, _ = attention_fp64(q, k[perm], v[perm], cu, 0.0884)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_brute_force_tiny():
    """T4: exact logits by fsum of exact bf16 products, exp/log in pure Python."""
    rng = np.random.default_rng(4)
    seqlens, H, D = [3, 7, 0, 6], 2, 8
    T = sum(seqlens)
    q, k, v = (rand_bits(rng, (T, H, D), scale=2.0) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    scale = 0.37
    out, lse, rows = attention_fp64(q, k, v, cu, scale)
    assert list(rows) == list(range(T))
    qf, kf, vf = (bf16_bits_to_f64(x).tolist() for x in (q, k, v))
    sigma = float(np.float32(scale))
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(H):
            for i in range(a, b):
                z = [sigma * math.fsum(qf[i][h][d] * kf[j][h][d] for d in range(D)) for j in range(a, b)]
                mz = max(z)
                w = [math.exp(t - mz) for t in z]
                s = math.fsum(w)
                assert abs(lse[h, i] - (mz + math.log(s))) <= 1e-12
                for d in range(D):
                    o = math.fsum(w[j - a] * vf[j][h][d] for j in range(a, b)) / s
                    assert abs(out[i, h, d] - o) <= 1e-13 * max(1.0, abs(o))


def test_segments_are_isolated():
    """T5: changing one segment's data leaves the other segments bit-identical."""
    rng = np.random.default_rng(5)
    cu = np.array([0, 40, 40, 90, 100])
    T, H, D = 100, 2, 16
    q, k, v = (rand_bits(rng, (T, H, D)) for _ in range(3))
    o1, l1, _ = attention_fp64(q, k, v, cu, 0.25)
    k2, v2 = k.copy(), v.copy()
    k2[40:90] = rand_bits(rng, (50, H, D))
    v2[40:90] = rand_bits(rng, (50, H, D))
    o2, l2, _ = attention_fp64(q, k2, v2, cu, 0.25)
    for a, b in [(0, 40), (90, 100)]:
        assert np.array_equal(o1[a:b], o2[a:b])
        assert np.array_equal(l1[:, a:b], l2[:, a:b])
    assert not np.array_equal(o1[40:90], o2[40:90])
    # a segment run alone equals the same rows inside the pack
    o3, l3, _ = attention_fp64(q[90:100], k[90:100], v[90:100], [0, 10], 0.25)
    assert np.array_equal(o3, o1[90:100]) and np.array_equal(l3, l1[:, 90:100])


def test_value_affine_map():
    """T6: O(a V + b) = a O(V) + b for exactly representable a V + b."""
    rng = np.random.default_rng(6)
    T, H, D = 50, 2, 8
    q, k = rand_bits(rng, (T, H, D)), rand_bits(rng, (T, H, D))
    vi = rng.integers(-4, 5, size=(T, H, D)).astype(np.float64)
    for a, b in [(2.0, 3.0), (-1.0, 0.0), (0.5, -7.0)]:
        o1, _, _ = attention_fp64(q, k, f64_to_bf16_bits(vi), [0, T], 0.5)
        o2, _, _ = attention_fp64(q, k, f64_to_bf16_bits(a * vi + b), [0, T], 0.5)
        np.testing.assert_allclose(o2, a * o1 + b, rtol=0, atol=1e-13)


def test_tiny_scale_limit():
    """T7: sigma = 2^-30 -> O ~ mean(V), LSE ~ ln L within sigma * max|q.k| bounds."""
    rng = np.random.default_rng(7)
    L, H, D = 300, 2, 128
    q, k, v = (rand_bits(rng, (L, H, D)) for _ in range(3))
    sigma = 2.0 ** -30
    out, lse, _ = attention_fp64(q, k, v, [0, L], sigma)
    qf, kf, vf = (bf16_bits_to_f64(x) for x in (q, k, v))
    for h in range(H):
        zmax = sigma * np.abs(qf[:, h] @ kf[:, h].T).max()
        bound_o = 2 * zmax * np.abs(vf[:, h]).max() * 2 + 1e-14
        np.testing.assert_allclose(out[:, h], np.broadcast_to(vf[:, h].mean(0), (L, D)), rtol=0, atol=bound_o)
        np.testing.assert_allclose(lse[h], math.log(L), rtol=0, atol=zmax + 1e-14)


def test_library_cross_check():
    """T8: torch's scaled_dot_product_attention in float64 on CPU, per segment."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    seqlens, H, D = [300, 77, 129], 3, 128
    T = sum(seqlens)
    q, k, v = (rand_bits(rng, (T, H, D)) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    scale = 1.0 / math.sqrt(128)
    out, lse, _ = attention_fp64(q, k, v, cu, scale)
    sigma = f32_to_f64(scale)
    for a, b in zip(cu[:-1], cu[1:]):
        qt, kt, vt = (torch.from_numpy(bf16_bits_to_f64(x[a:b])).permute(1, 0, 2).contiguous() for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sigma)
        np.testing.assert_allclose(out[a:b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)
        ref_lse = torch.logsumexp((qt @ kt.transpose(1, 2)) * sigma, dim=-1)
        np.testing.assert_allclose(lse[:, a:b], ref_lse.numpy(), rtol=0, atol=1e-10)


def test_single_key_segment():
    """A one-token segment: O = v, LSE = sigma q.k."""
    rng = np.random.default_rng(9)
    q, k, v = (rand_bits(rng, (1, 4, 128)) for _ in range(3))
    out, lse, _ = attention_fp64(q, k, v, [0, 1], 0.125)
    qf, kf, vf = (bf16_bits_to_f64(x) for x in (q, k, v))
    np.testing.assert_array_equal(out, vf)
    for h in range(4):
        assert abs(lse[h, 0] - 0.125 * math.fsum(qf[0, h] * kf[0, h])) < 1e-13


def test_scale_is_the_fp32_value():
    """The oracle uses the fp32 rounding of the scale it is given (the value the ABI carries)."""
    assert f32_to_f64(0.1) == float(np.float32(0.1)) != 0.1
    assert f32_to_f64(1 / math.sqrt(128)) == 0.0883883461356163
    rng = np.random.default_rng(10)
    q, k, v = (rand_bits(rng, (20, 1, 8)) for _ in range(3))
    o1, l1, _ = attention_fp64(q, k, v, [0, 20], 0.1)
    o2, l2, _ = attention_fp64(q, k, v, [0, 20], float(np.float32(0.1)))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_subset_matches_full():
    rng = np.random.default_rng(11)
    cu = [0, 30, 130]
    q, k, v = (rand_bits(rng, (130, 2, 16)) for _ in range(3))
    o, l, _ = attention_fp64(q, k, v, cu, 0.2)
    rows = np.array([0, 5, 29, 30, 77, 129])
    os_, ls, r = attention_fp64(q, k, v, cu, 0.2, rows=rows)
    assert np.array_equal(r, rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls, l[:, rows])
    o1, l1, _ = attention_fp64(q, k, v, cu, 0.2, workers=1)
    assert np.array_equal(o1, o) and np.array_equal(l1, l)


def test_empty_inputs_and_bad_arguments():
    q = np.zeros((0, 2, 8), dtype=np.uint16)
    out, lse, rows = attention_fp64(q, q, q, [0], 0.1)
    assert out.shape == (0, 2, 8) and lse.shape == (2, 0)
    out, lse, rows = attention_fp64(q, q, q, [0, 0, 0], 0.1)
    assert out.shape == (0, 2, 8)
    z = np.zeros((4, 1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        attention_fp64(z, z, z, [0, 5], 0.1)
    with pytest.raises(ValueError):
        attention_fp64(z, z, z, [0, 3, 2], 0.1)
    with pytest.raises(ValueError):
        attention_fp64(z, z, z, [1, 3], 0.1)
    with pytest.raises(ValueError):
        attention_fp64(z, z, z, [0, 2], 0.1, rows=np.array([3]))
