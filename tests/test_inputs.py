"""The seeded input generator: definition, determinism, statistics, conditioning."""

import math

import numpy as np
import pytest

from long_sequence_video_amd import inputs as gen


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
    return z ^ (z >> 31)


def _splitmix_stream(seed, n):
    """The published splitmix64 generator, stepped sequentially from state ``seed``."""
    state, out = seed, []
    for _ in range(n):
        state = (state + GAMMA) & MASK
        out.append(_mix(state))
    return out


def _bf16_rne(x: float) -> int:
    u = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF


def test_matches_published_definition():
    seed, tensor = 1234, 2
    s0 = _splitmix_stream(seed, tensor + 1)[tensor]
    words = _splitmix_stream(s0, 12)
    got = gen.normal_bf16(11, seed, tensor)
    for e in range(11):
        a, b = words[2 * (e // 2)], words[2 * (e // 2) + 1]
        u1 = ((a >> 11) + 1) * 2.0 ** -53
        u2 = (b >> 11) * 2.0 ** -53
        r, t = math.sqrt(-2 * math.log(u1)), 2 * math.pi * u2
        z = r * math.cos(t) if e % 2 == 0 else r * math.sin(t)
        assert abs(gen.normal_f64_at(seed, tensor, e) - z) < 1e-12
        assert got[e] == _bf16_rne(z)


def test_deterministic_and_thread_independent():
    import subprocess
    import sys
    a = gen.normal_bf16(100_001, 7, 0)
    b = gen.normal_bf16(100_001, 7, 0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, gen.normal_bf16(100_001, 7, 1))
    assert not np.array_equal(a, gen.normal_bf16(100_001, 8, 0))
    code = ("import numpy as np, sys; from long_sequence_video_amd import inputs as g; "
            "sys.stdout.write(g.normal_bf16(100001, 7, 0).tobytes().hex()[:4000] + "
            "str(int(g.normal_bf16(100001, 7, 0).astype(np.int64).sum())))")
    import os
    env = dict(os.environ, OMP_NUM_THREADS="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out1 = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True, check=True)
    env["OMP_NUM_THREADS"] = "5"
    out5 = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True, check=True)
    assert out1.stdout == out5.stdout
    assert out1.stdout.endswith(str(int(a.astype(np.int64).sum())))


def test_normal_moments():
    x = gen.normal_bf16(1 << 20, 99, 1).astype(np.uint32) << 16
    f = x.view(np.float32).astype(np.float64)
    n = f.size
    assert abs(f.mean()) < 5 / math.sqrt(n)
    assert abs(f.var() - 1) < 0.01
    assert abs((f ** 4).mean() - 3) < 0.05
    assert np.isfinite(f).all()


def test_rms_normalized_rows():
    inp = gen.generate([100], heads=3, seed=5, rms_qk=True)
    for t in (inp.q, inp.k):
        f = (t.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ms = (f ** 2).mean(-1)
        assert np.all(np.abs(ms - 1) < 2e-2)
    raw = gen.generate([100], heads=3, seed=5)
    assert np.array_equal(raw.v, inp.v)  # V is not normalised


def test_k_boost_rows_are_exact_multiples():
    inp = gen.generate([4096], heads=2, seed=1002, k_boost_frac=0.01)
    raw = gen.generate([4096], heads=2, seed=1002)
    rows = inp.meta["k_boost_row_ids"]
    assert len(rows) == 41 and len(set(rows.tolist())) == 41
    f = lambda t: (t.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(inp.k[rows]), 8 * f(raw.k[rows]))
    mask = np.ones(4096, bool)
    mask[rows] = False
    assert np.array_equal(inp.k[mask], raw.k[mask])
    assert np.array_equal(inp.q, raw.q) and np.array_equal(inp.v, raw.v)


def test_choose_rows_distinct_and_seeded():
    a = gen.choose_rows(50, 1000, 3)
    assert len(set(a.tolist())) == 50 and a.min() >= 0 and a.max() < 1000
    assert np.all(np.diff(a) > 0)
    assert np.array_equal(a, gen.choose_rows(50, 1000, 3))
    assert not np.array_equal(a, gen.choose_rows(50, 1000, 4))
    assert np.array_equal(gen.choose_rows(10, 10, 1), np.arange(10))


def test_config_shapes_and_flops():
    shapes = {
        "tiny_s256_h4": ([256], 4),
        "s4096_h56_kboost": ([4096], 56),
        "sp4_share_s19394_h14": ([19394], 14),
        "h3_s38000_h56": ([38000], 56),
        "varlen_19394_38000_104000_h56": ([19394, 38000, 104000], 56),
    }
    assert set(shapes) == set(gen.CONFIGS)
    for name, (seqlens, heads) in shapes.items():
        cfg = gen.CONFIGS[name]
        assert cfg["seqlens"] == seqlens and cfg["heads"] == heads
    tiny = gen.make_config("tiny_s256_h4")
    assert tiny.q.shape == (256, 4, 128) and list(tiny.cu_seqlens) == [0, 256]
    assert tiny.flops() == 4 * 256 ** 2 * 4 * 128
    assert tiny.scale == 1 / math.sqrt(128)


def test_generate_arguments():
    with pytest.raises(ValueError):
        gen.generate([-1], heads=1, seed=0)
    with pytest.raises(ValueError):
        gen.generate([10], heads=1, seed=0, total_tokens=5)
    x = gen.generate([3, 0, 4], heads=2, head_dim=8, seed=0, total_tokens=9)
    assert x.q.shape == (9, 2, 8) and list(x.cu_seqlens) == [0, 3, 3, 7]
    assert x.max_seqlen == 4 and x.seqlens == [3, 0, 4]


def test_low_first_tile_sets_channel_zero_only():
    """Channel 0: q = 8 everywhere, k = -c on each segment's first 256 keys and +c elsewhere
    (also past cu[-1]); every other channel equals the plain draw."""
    plain = gen.generate([300, 0, 40, 600], heads=2, seed=5, total_tokens=950)
    low = gen.generate([300, 0, 40, 600], heads=2, seed=5, total_tokens=950, low_first_tile=80.0)
    assert np.array_equal(low.q[:, :, 1:], plain.q[:, :, 1:]) and np.array_equal(low.v, plain.v)
    assert np.array_equal(low.k[:, :, 1:], plain.k[:, :, 1:])
    assert np.all(bf16_to_f64(low.q[:, :, 0]) == 8.0)
    k0 = bf16_to_f64(low.k[:, :, 0])
    first = np.zeros(950, bool)
    first[0:256] = first[300:340] = first[340:596] = True
    assert np.all(k0[first] == -80.0) and np.all(k0[~first] == 80.0)
    assert low.meta["low_first_tile"] == 80.0


def test_c_e4m3_quantiser_equals_the_numpy_definition():
    """The C quantiser (used for the FP8 workloads) gives the same bytes as
    ``f64_to_e4m3_bits(x / descale)`` on random values and on the edge cases: zeros of both
    signs, ties between two e4m3 values (to even), the subnormal range, saturation at 448."""
    rng = np.random.default_rng(5)
    x = gen.normal_bf16(200_000, 77, 0)
    edges = np.array([0.0, -0.0, 448.0, -448.0, 460.0, 464.0, 1e6, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10,
                      1.5 * 2.0 ** -10, 1.0625, 1.1875, 3.0 * 2.0 ** -11, 17.0, 19.0, 240.0, 232.0, 248.0])
    ebits = gen.f64_to_bf16_bits(np.r_[edges, -edges])
    for descale in (1.0, 0.0123, float(np.float32(5.61 / 448.0)), 2.0 ** -7, 3.7):
        for bits in (x, ebits, rng.integers(0, 0x7F80, 5000).astype(np.uint16)):
            vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            want = gen.f64_to_e4m3_bits(vals / descale)
            got = gen.quantize_e4m3_bf16(bits, descale)
            assert np.array_equal(got, want), (descale, np.flatnonzero(got != want)[:5])


def test_c_amax_equals_numpy():
    x = gen.normal_bf16(100_001, 3, 1)
    vals = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert gen.amax_bf16(x) == np.abs(vals).max()
    assert gen.amax_bf16(np.zeros(0, np.uint16)) == 0.0


def test_varlen_rope_tables_restart_per_segment():
    """Each segment's tokens take positions 0, 1, ... of their own sequence: the first token of
    every segment has cos 1 and sin 0, and a segment's rows equal the single-sequence table."""
    seqlens = [5, 0, 9, 3]
    cos, sin = gen.rope_tables_varlen(seqlens, 32)
    assert cos.shape == (17, 32) and sin.shape == (17, 32)
    one, zero = gen.f64_to_bf16_bits(1.0), gen.f64_to_bf16_bits(0.0)
    for a in (0, 5, 14):
        assert np.all(cos[a] == one) and np.all(sin[a] == zero)
    c9, s9 = gen.rope_tables(9, 32)
    assert np.array_equal(cos[5:14], c9) and np.array_equal(sin[5:14], s9)
