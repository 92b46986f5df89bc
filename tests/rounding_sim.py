"""fp64 simulations of the kernels' roundings, from which the GPU tests' tolerances are derived.

Test infrastructure. Each function redoes one kernel's arithmetic in numpy with the kernel's
own rounding steps (bf16 / fp32 / e4m3 roundings at the points where the kernel rounds, the
order in which it sums where that matters), so that its distance from the exact fp64 oracle
is the error the kernel is expected to make. The simulations import nothing from the HIP
path and are not the oracle: the oracle is the plain definition; these are models of an
implementation, used only to size the bars.
"""

from __future__ import annotations

import numpy as np

from oracle import bf16_bits_to_f64, e4m3_bits_to_f64


def f32(x):
    """Round to fp32 (nearest even), back in fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to fp32, then to bf16 (nearest even), back in fp64: the kernels' bf16 casts."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bf16_bits_to_f64(bits)


def e4m3(x):
    """Round to OCP e4m3 (nearest even in the binade, subnormal spacing 2^-9), no saturation
    needed here (callers keep |x| <= 2^8)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = 2.0 ** (e - 3)
    return np.sign(x) * np.round(a / quantum) * quantum


# ---------------------------------------------------------------------------- backward


def bwd_sim(q_bits, k_bits, v_bits, do_bits, o_bits, lse32, scale):
    """The backward kernels' arithmetic for one segment and head ([L, 128] bf16 bit arrays, the
    bf16 O and fp32 LSE it is handed):

    * prep: -LSE / scale and D = dO . O (bf16 O) in fp32;
    * S = Q K^T from exact bf16 products, accumulated in fp32, started at -LSE / scale;
      P = exp2(fp32(scale log2 e) S') in fp32;
    * dP' = dO V^T - D in fp32; dS = P dP' in fp32;
    * P and dS rounded to bf16 for the products dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K,
      accumulated in fp32, rounded to bf16.
    fp32 accumulation of a product is modelled as the exact sum rounded once to fp32 (its own
    error, ~2^-24 relative per term at these sizes, is far below the bf16 roundings).
    Returns (dq, dk, dv) in fp64 (bf16 values).
    """
    q, k, v, do, o = (bf16_bits_to_f64(x) for x in (q_bits, k_bits, v_bits, do_bits, o_bits))
    sc = float(np.float32(scale))
    c = float(np.float32(sc * np.log2(np.e)))
    nl = f32(-f32(lse32) * f32(1.0 / sc))                    # -LSE / scale
    dvec = f32(np.sum(do * o, axis=1))                       # D = dO . O (bf16 O)
    s = f32(q @ k.T + nl[:, None])                           # S' = S - LSE / scale
    p = f32(np.exp2(f32(c * s)))
    dp = f32(do @ v.T - dvec[:, None])                       # dP' = dP - D
    ds = f32(p * dp)
    pb, dsb = bf16(p), bf16(ds)
    dv = bf16(f32(pb.T @ do))
    dk = bf16(sc * f32(dsb.T @ q))
    dq = bf16(sc * f32(dsb @ k))
    return dq, dk, dv


def bwd_errors(inp, do_bits, o_ref, lse_ref, grads_ref):
    """Normalised errors (the GPU test's measure) of bwd_sim against the oracle's gradients on
    every segment and head of ``inp``: max |G - G_ref| / max |G_ref| and mean |G - G_ref| /
    mean |G_ref| per gradient tensor."""
    o_bits = None
    from long_sequence_video_amd import inputs as gen
    o_bits = gen.f64_to_bf16_bits(o_ref)
    lse32 = lse_ref.astype(np.float32)
    sims = {n: np.zeros_like(grads_ref[n]) for n in ("dq", "dk", "dv")}
    cu = inp.cu_seqlens
    for a, b in zip(cu[:-1], cu[1:]):
        for h in range(inp.n_heads):
            dq, dk, dv = bwd_sim(inp.q[a:b, h], inp.k[a:b, h], inp.v[a:b, h], do_bits[a:b, h], o_bits[a:b, h],
                                 lse32[h, a:b], inp.scale)
            sims["dq"][a:b, h], sims["dk"][a:b, h], sims["dv"][a:b, h] = dq, dk, dv
    out = {}
    for n in ("dq", "dk", "dv"):
        err = np.abs(sims[n] - grads_ref[n])
        r = np.abs(grads_ref[n])
        out[n] = (float(err.max() / r.max()), float(err.mean() / r.mean()))
    return out


# ---------------------------------------------------------------------------- FP8 forward

_SIM_SRC = __import__("os").path.join(__import__("os").path.dirname(__file__), "fp8_sim.c")
_SIM_LIB = __import__("os").path.join(__import__("os").path.dirname(__file__), "libfp8sim.so")
_sim = None


def _fp8_lib():
    """Builds tests/fp8_sim.c with gcc on first use (plain C, OpenMP)."""
    import ctypes
    import os
    import subprocess
    global _sim
    if _sim is not None:
        return _sim
    if not os.path.exists(_SIM_LIB) or os.path.getmtime(_SIM_LIB) < os.path.getmtime(_SIM_SRC):
        tmp = "%s.%d.tmp" % (_SIM_LIB, os.getpid())  # one name per process: parallel test workers
        subprocess.run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Werror",
                        "-ffp-contract=off", "-o", tmp, _SIM_SRC, "-lm"], check=True)
        os.replace(tmp, _SIM_LIB)
    lib = ctypes.CDLL(_SIM_LIB)
    p = ctypes.c_void_p
    lib.fp8_fwd_sim.argtypes = [p, p, p, ctypes.c_int64, ctypes.c_int64, p, ctypes.c_int, p, ctypes.c_int,
                                ctypes.c_float, ctypes.c_float, ctypes.c_int, p, p]
    lib.fp8_fwd_sim.restype = ctypes.c_int
    _sim = lib
    return lib


def fp8_fwd_sim(f8, heads=None, zero_counts=False):
    """The FP8 kernel's arithmetic (``tests/fp8_sim.c``) on ``f8`` (an ``inputs.Fp8Inputs``) for
    ``heads`` (default: all). Returns (O bf16 bits [T, n_heads_sel, 128], LSE fp32 [n_sel, T])."""
    import ctypes
    lib = _fp8_lib()
    hs = np.arange(f8.n_heads, dtype=np.int32) if heads is None else np.asarray(heads, dtype=np.int32)
    T, H = f8.total_tokens, f8.n_heads
    q, k, v = (np.ascontiguousarray(x, dtype=np.uint8) for x in (f8.q, f8.k, f8.v))
    cu = np.ascontiguousarray(f8.cu_seqlens, dtype=np.int32)
    # as the library computes it from the fp32 arguments it is passed
    c = np.float32(float(np.float32(f8.scale)) * float(np.float32(f8.descale_q)) * float(np.float32(f8.descale_k)) *
                   1.4426950408889634074)
    o = np.zeros((T, len(hs), 128), np.uint16)
    lse = np.zeros((len(hs), T), np.float32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = lib.fp8_fwd_sim(ptr(q), ptr(k), ptr(v), T, H, ptr(cu), len(cu) - 1, ptr(hs), len(hs), c,
                         np.float32(f8.descale_v), int(zero_counts), ptr(o), ptr(lse))
    if rc != 0:
        raise RuntimeError(f"fp8_fwd_sim failed ({rc})")
    return o, lse
