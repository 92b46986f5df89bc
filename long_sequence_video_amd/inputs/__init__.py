"""Seeded synthetic inputs for the attention forward (bf16 bit patterns).

The arrays this module returns feed both the HIP library and the fp64 oracle;
it holds none of the attention arithmetic. The generator itself is C
(``gen.c``, built into ``liblsvgen.so``), counter-based, so results do not
depend on the number of threads. See ``gen.c`` for the exact definitions.

Workloads stand in for the MiniMax-H3 packed clips the pages describe
(TensorRT-LLM PR #21275, Description and Measurements: 19k / 38k / 104k-token
blocks with 56 heads x 128; the 544x960x124 clip packs to 19,394 tokens;
FastVideo perf/ulysses-h3-adaptive commit message: sp=4 gives one rank 14 of
the 56 heads). Tensor ids: Q = 0, K = 1, V = 2, boosted-K row choice = 3.

The QKV-prologue inputs (FastVideo #2049, MotionKernel ``qkv_prologue`` and its
tests) add per-head norm weights (ids 4, 5) and cos/sin tables: either the usual
rotate-half RoPE angles, or iid N(0,1) tables (ids 6, 7) as the page's own
kernel test draws them.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsvgen.so")
SOURCE_PATH = os.path.join(_HERE, "gen.c")

Q_ID, K_ID, V_ID, CHOOSE_ID = 0, 1, 2, 3
QW_ID, KW_ID, COS_ID, SIN_ID = 4, 5, 6, 7
RMS_EPS = 1e-5  # the H3 QK-norm eps (FastVideo #2049, MotionKernel qkv prologue)

_lib = None


def build_library(verbose: bool = False) -> str:
    """Compile ``gen.c`` with gcc into ``liblsvgen.so`` (always recompiles)."""
    import subprocess
    tmp = "%s.%d.tmp" % (LIB_PATH, os.getpid())  # one name per process: concurrent builds
    include = os.path.join(os.path.dirname(os.path.dirname(_HERE)), "include")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11", "-Wall", "-Werror",
           "-I", include, SOURCE_PATH, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build_library()
    lib = ctypes.CDLL(LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.lsvgen_normal_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32]
    lib.lsvgen_rms_normalize_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double]
    lib.lsvgen_choose.argtypes = [i64p, ctypes.c_int64, ctypes.c_int64, i64p, ctypes.c_uint64, ctypes.c_uint32]
    lib.lsvgen_scale_rows_bf16.argtypes = [u16p, i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_float]
    lib.lsvgen_normal_f64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64]
    lib.lsvgen_normal_f64_at.restype = ctypes.c_double
    lib.lsvgen_quantize_e4m3_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_uint8)]
    lib.lsvgen_amax_bf16.argtypes = [u16p, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)]
    for f in (lib.lsvgen_normal_bf16, lib.lsvgen_rms_normalize_bf16, lib.lsvgen_choose,
              lib.lsvgen_scale_rows_bf16, lib.lsvgen_quantize_e4m3_bf16, lib.lsvgen_amax_bf16):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what}: invalid arguments")


def normal_bf16(n: int, seed: int, tensor: int) -> np.ndarray:
    """``n`` bf16 standard normals (uint16 bit patterns) of stream (seed, tensor)."""
    out = np.empty(n, dtype=np.uint16)
    lib = _load()
    _check(lib.lsvgen_normal_bf16(out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), n, seed, tensor),
           "normal_bf16")
    return out


def normal_f64_at(seed: int, tensor: int, e: int) -> float:
    """Element ``e`` of stream (seed, tensor) before rounding (for tests)."""
    return _load().lsvgen_normal_f64_at(seed, tensor, e)


def rms_normalize_rows(x: np.ndarray, eps: float = RMS_EPS) -> None:
    """In place: every last-axis row ``x <- bf16(x * (mean(x^2) + eps)^-1/2)``."""
    if x.dtype != np.uint16 or not x.flags.c_contiguous:
        raise ValueError("expected a C-contiguous uint16 array")
    d = x.shape[-1]
    _check(_load().lsvgen_rms_normalize_bf16(x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                             x.size // d, d, eps), "rms_normalize_rows")


def choose_rows(n_choose: int, n_total: int, seed: int, tensor: int = CHOOSE_ID) -> np.ndarray:
    """``n_choose`` distinct sorted indices in ``[0, n_total)`` (partial Fisher-Yates)."""
    out = np.empty(n_choose, dtype=np.int64)
    work = np.empty(max(n_total, 1), dtype=np.int64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    _check(_load().lsvgen_choose(out.ctypes.data_as(i64p), n_choose, n_total, work.ctypes.data_as(i64p),
                                 seed, tensor), "choose_rows")
    return out


def scale_rows(x: np.ndarray, rows: np.ndarray, factor: float) -> None:
    """In place: multiply token rows ``rows`` of ``x`` ([T, ...], uint16 bf16) by ``factor``."""
    if x.dtype != np.uint16 or not x.flags.c_contiguous:
        raise ValueError("expected a C-contiguous uint16 array")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= x.shape[0]):
        raise ValueError("row index out of range")
    row_len = x.size // x.shape[0]
    _check(_load().lsvgen_scale_rows_bf16(x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                          rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          rows.size, row_len, factor), "scale_rows")


@dataclass
class Inputs:
    """One attention workload: packed bf16 q/k/v and its segment boundaries."""
    name: str
    q: np.ndarray           # uint16 [total, heads, head_dim]
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: np.ndarray  # int32 [n_seqs + 1]
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def seqlens(self) -> list[int]:
        cu = self.cu_seqlens.astype(np.int64)
        return [int(b - a) for a, b in zip(cu[:-1], cu[1:])]

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens, default=0)

    def flops(self) -> float:
        """Attention forward flops counted as sum over sequences of 4 * S^2 * H * D."""
        return float(sum(4.0 * s * s * self.n_heads * self.head_dim for s in self.seqlens))


def generate(seqlens, heads: int, head_dim: int = 128, *, seed: int, rms_qk: bool = False,
             k_boost_frac: float = 0.0, k_boost_factor: float = 8.0, scale: float | None = None,
             low_first_tile: float = 0.0, name: str = "custom", total_tokens: int | None = None) -> Inputs:
    """Packed inputs for segments of lengths ``seqlens``.

    * q, k, v: iid N(0,1) rounded to bf16, streams (seed, 0/1/2), row-major
      ``[total, heads, head_dim]``.
    * ``rms_qk``: every (token, head) row of q and k is RMS-normalised (unit
      weight, eps 1e-5) in double and rounded to bf16.
    * ``k_boost_frac``: ``round(frac * total)`` token rows of k, chosen by the
      (seed, 3) stream, are multiplied by ``k_boost_factor`` on every head.
    * ``low_first_tile`` = c > 0: channel 0 of every q row is set to 8 and channel 0 of every
      k row to +c, except the first 256 keys of each segment, which get -c (bf16 exact for
      the values used). Every query then scores about 16 c * scale below the rest on its
      segment's first key tile: the input on which a softmax that fixes its reference at the
      first tile's maximum must fall back everywhere.
    * ``scale`` defaults to ``1/sqrt(head_dim)``.
    * ``total_tokens`` may exceed ``sum(seqlens)``; the extra rows are generated
      too but lie outside every segment.
    """
    seqlens = [int(s) for s in seqlens]
    if any(s < 0 for s in seqlens):
        raise ValueError("negative sequence length")
    used = sum(seqlens)
    total = used if total_tokens is None else int(total_tokens)
    if total < used:
        raise ValueError("total_tokens smaller than the sum of seqlens")
    shape = (total, heads, head_dim)
    n = total * heads * head_dim
    q = normal_bf16(n, seed, Q_ID).reshape(shape)
    k = normal_bf16(n, seed, K_ID).reshape(shape)
    v = normal_bf16(n, seed, V_ID).reshape(shape)
    meta = {"seed": seed, "rms_qk": rms_qk, "k_boost_rows": 0}
    if rms_qk:
        rms_normalize_rows(q)
        rms_normalize_rows(k)
    if k_boost_frac > 0:
        nb = int(round(k_boost_frac * total))
        rows = choose_rows(nb, total, seed)
        scale_rows(k, rows, k_boost_factor)
        meta["k_boost_rows"] = nb
        meta["k_boost_row_ids"] = rows
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    if low_first_tile > 0:
        lift = f64_to_bf16_bits(np.array([low_first_tile, -low_first_tile, 8.0]))
        q[:, :, 0] = lift[2]
        k[:, :, 0] = lift[0]
        for a, b in zip(cu[:-1], cu[1:]):
            k[a:min(b, a + 256), :, 0] = lift[1]
        meta["low_first_tile"] = float(low_first_tile)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    return Inputs(name, q, k, v, cu, sc, meta)


# The five workloads (tokens x heads x 128, bf16, seeds 1001..1005).
CONFIGS = {
    "tiny_s256_h4": dict(seqlens=[256], heads=4, seed=1001),
    "s4096_h56_kboost": dict(seqlens=[4096], heads=56, seed=1002, k_boost_frac=0.01),
    "sp4_share_s19394_h14": dict(seqlens=[19394], heads=14, seed=1003, rms_qk=True),
    "h3_s38000_h56": dict(seqlens=[38000], heads=56, seed=1004, rms_qk=True),
    "varlen_19394_38000_104000_h56": dict(seqlens=[19394, 38000, 104000], heads=56, seed=1005),
}


def make_config(name: str) -> Inputs:
    """Inputs of one of the named workloads in ``CONFIGS``."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    return generate(name=name, **CONFIGS[name])


# ---------------------------------------------------------------- QKV prologue inputs


def f64_to_bf16_bits(x) -> np.ndarray:
    """fp64 -> fp32 (round to nearest even) -> bf16 bits (round to nearest even)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rope_tables(seq_len: int, rotary_dim: int, *, base: float = 10000.0, start: int = 0):
    """cos/sin tables ``[S, R]`` (bf16 bits) in the rotate-half layout: channels i and
    i + R/2 share the angle ``(start + s) * base^(-2 i / R)``."""
    if rotary_dim % 2:
        raise ValueError("rotary_dim must be even")
    h = rotary_dim // 2
    inv_freq = base ** (-2.0 * np.arange(h, dtype=np.float64) / max(rotary_dim, 1))
    ang = (start + np.arange(seq_len, dtype=np.float64))[:, None] * inv_freq[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return f64_to_bf16_bits(np.cos(ang)), f64_to_bf16_bits(np.sin(ang))


def rope_tables_varlen(seqlens, rotary_dim: int, *, base: float = 10000.0):
    """Per-token cos/sin tables ``[sum(seqlens), R]`` (bf16 bits) for a varlen pack: each
    segment's tokens take the positions 0, 1, ... of their own sequence."""
    cs, ss = [], []
    for n in seqlens:
        c, s = rope_tables(int(n), rotary_dim, base=base)
        cs.append(c)
        ss.append(s)
    if not cs:
        return np.zeros((0, rotary_dim), np.uint16), np.zeros((0, rotary_dim), np.uint16)
    return np.concatenate(cs), np.concatenate(ss)


@dataclass
class QNormInputs:
    """A forward with the QKV prologue in front of it: raw q, k, v [T, H, 128], bf16 norm weights
    [128] and per-token cos/sin tables [T, R] (bf16 bits), and the segment boundaries."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_weight: np.ndarray
    k_weight: np.ndarray
    cos: np.ndarray
    sin: np.ndarray
    cu_seqlens: np.ndarray
    scale: float
    eps: float = RMS_EPS

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def rotary_dim(self) -> int:
        return int(self.cos.shape[1])

    @property
    def seqlens(self) -> list[int]:
        cu = self.cu_seqlens.astype(np.int64)
        return [int(b - a) for a, b in zip(cu[:-1], cu[1:])]

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens, default=0)

    def flops(self) -> float:
        return float(sum(4.0 * s * s * self.n_heads * self.q.shape[2] for s in self.seqlens))


def generate_qnorm(seqlens, heads: int, rotary_dim: int = 96, *, seed: int, tables: str = "rope",
                   name: str = "qnorm") -> QNormInputs:
    """Raw q, k, v iid N(0,1) (streams (seed, 0/1/2)), norm weights iid N(0,1) (streams 4, 5) and
    per-token tables: RoPE angles of each token's position in its segment (``"rope"``) or iid
    N(0,1) (``"normal"``, streams 6, 7), for a varlen pack of ``seqlens``."""
    inp = generate(seqlens, heads, seed=seed, name=name)
    qw = normal_bf16(128, seed, QW_ID)
    kw = normal_bf16(128, seed, KW_ID)
    t = inp.total_tokens
    if tables == "rope":
        cos, sin = rope_tables_varlen(inp.seqlens, rotary_dim)
    elif tables == "normal":
        cos = normal_bf16(t * rotary_dim, seed, COS_ID).reshape(t, rotary_dim)
        sin = normal_bf16(t * rotary_dim, seed, SIN_ID).reshape(t, rotary_dim)
    else:
        raise ValueError("tables must be 'rope' or 'normal'")
    return QNormInputs(name, inp.q, inp.k, inp.v, qw, kw, cos, sin, inp.cu_seqlens, inp.scale)


@dataclass
class PrologueInputs:
    """One QKV-prologue workload (bf16 bit patterns)."""
    name: str
    q: np.ndarray          # uint16 [B, S, H, D]
    k: np.ndarray
    v: np.ndarray
    q_weight: np.ndarray   # uint16 [D]
    k_weight: np.ndarray
    cos: np.ndarray        # uint16 [S, R]
    sin: np.ndarray
    eps: float
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        return tuple(int(x) for x in self.q.shape)

    @property
    def rotary_dim(self) -> int:
        return int(self.cos.shape[1])

    def algorithmic_bytes(self) -> int:
        """HBM bytes of one pass: q, k, v read and the three planes written once (bf16),
        plus the cos/sin rows and the two weights."""
        b, s, h, d = self.shape
        return 6 * b * s * h * d * 2 + 2 * s * self.rotary_dim * 2 + 2 * d * 2


def generate_prologue(batch: int, seq_len: int, heads: int, head_dim: int = 128, rotary_dim: int = 96, *,
                      seed: int, tables: str = "rope", eps: float = RMS_EPS, name: str = "prologue") -> PrologueInputs:
    """q, k, v iid N(0,1) ``[B, S, H, D]`` (streams (seed, 0/1/2)); norm weights iid N(0,1)
    (streams 4, 5; the page's test draws them so, which also covers negative weights);
    ``tables="rope"``: RoPE angles from position 0, ``"normal"``: iid N(0,1) tables
    (streams 6, 7)."""
    shape = (batch, seq_len, heads, head_dim)
    n = batch * seq_len * heads * head_dim
    q = normal_bf16(n, seed, Q_ID).reshape(shape)
    k = normal_bf16(n, seed, K_ID).reshape(shape)
    v = normal_bf16(n, seed, V_ID).reshape(shape)
    qw = normal_bf16(head_dim, seed, QW_ID)
    kw = normal_bf16(head_dim, seed, KW_ID)
    if tables == "rope":
        cos, sin = rope_tables(seq_len, rotary_dim)
    elif tables == "normal":
        cos = normal_bf16(seq_len * rotary_dim, seed, COS_ID).reshape(seq_len, rotary_dim)
        sin = normal_bf16(seq_len * rotary_dim, seed, SIN_ID).reshape(seq_len, rotary_dim)
    else:
        raise ValueError("tables must be 'rope' or 'normal'")
    return PrologueInputs(name, q, k, v, qw, kw, cos, sin, float(eps), {"seed": seed, "tables": tables})


# QKV-prologue workloads: the page's kernel-test shape (512 tokens, random tables), the
# varlen pack's 161,394 tokens as one [1, S] sequence with RoPE tables (the bench
# workload), and the page's int32-plane test shape (4 x 40,000 x 56 x 128).
PROLOGUE_CONFIGS = {
    "prologue_s512_h56_randtab": dict(batch=1, seq_len=512, heads=56, seed=2001, tables="normal"),
    "prologue_s161394_h56": dict(batch=1, seq_len=161394, heads=56, seed=2002),
    "prologue_b4_s40000_h56": dict(batch=4, seq_len=40000, heads=56, seed=2003, tables="normal"),
}


def make_prologue_config(name: str) -> PrologueInputs:
    if name not in PROLOGUE_CONFIGS:
        raise KeyError(f"unknown prologue workload {name!r}; known: {sorted(PROLOGUE_CONFIGS)}")
    return generate_prologue(name=name, **PROLOGUE_CONFIGS[name])


# ---------------------------------------------------------------- FP8 (e4m3) attention inputs

E4M3_MAX = 448.0


def f64_to_e4m3_bits(x) -> np.ndarray:
    """Quantise to OCP FP8 e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
    infinities): round to nearest even, subnormals below 2^-6, saturation at +-448."""
    x = np.asarray(x, dtype=np.float64)
    sign = (x < 0) | ((x == 0) & np.signbit(x))
    a = np.minimum(np.abs(x), E4M3_MAX)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    q = 2.0 ** (e - 3)                       # spacing of the binade (subnormals: 2^-9)
    r = np.minimum(np.round(a / q) * q, E4M3_MAX)   # numpy rounds half to even
    # encode r exactly
    ee = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, ee + 7, 0).astype(np.int64)
    mant = np.where(normal, r / 2.0 ** ee - 1.0, r / 2.0 ** -9 / 8.0) * 8.0
    mant = np.rint(mant).astype(np.int64)
    bits = (exp_field << 3) | mant
    bits = np.where(r == 0, 0, bits)
    return (bits | (sign.astype(np.int64) << 7)).astype(np.uint8)


@dataclass
class Fp8Inputs:
    """One FP8 attention workload: e4m3 q/k/v bytes with per-tensor descales (fp32)."""
    name: str
    q: np.ndarray           # uint8 [total, heads, head_dim]
    k: np.ndarray
    v: np.ndarray
    descale_q: float
    descale_k: float
    descale_v: float
    cu_seqlens: np.ndarray
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def seqlens(self) -> list[int]:
        cu = self.cu_seqlens.astype(np.int64)
        return [int(b - a) for a, b in zip(cu[:-1], cu[1:])]

    @property
    def max_seqlen(self) -> int:
        return max(self.seqlens, default=0)

    def flops(self) -> float:
        return float(sum(4.0 * s * s * self.n_heads * self.q.shape[2] for s in self.seqlens))


def amax_bf16(bits: np.ndarray) -> float:
    """The largest |x| of a bf16 array (uint16 bit patterns)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = ctypes.c_double()
    _check(_load().lsvgen_amax_bf16(b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), b.size, ctypes.byref(out)),
           "amax_bf16")
    return out.value


def quantize_e4m3_bf16(bits: np.ndarray, descale: float) -> np.ndarray:
    """e4m3 bits of bf16 values / descale (the C generator; equal to
    ``f64_to_e4m3_bits(x / descale)``, without float64 temporaries), same shape."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.uint8)
    _check(_load().lsvgen_quantize_e4m3_bf16(b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), b.size,
                                               float(descale), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))),
           "quantize_e4m3_bf16")
    return out


def quantize_fp8(inp: Inputs, name: str | None = None) -> Fp8Inputs:
    """Per-tensor e4m3 quantisation of a bf16 workload: descale = fp32(amax / 448), values
    x / descale rounded to e4m3 (the usual amax recipe for FP8 attention inputs)."""
    out = {}
    for key in ("q", "k", "v"):
        bits = getattr(inp, key)
        amax = amax_bf16(bits) or 1.0
        d = float(np.float32(amax / E4M3_MAX))
        out[key] = (quantize_e4m3_bf16(bits, d), d)
    return Fp8Inputs(name or inp.name + "_fp8", out["q"][0], out["k"][0], out["v"][0], out["q"][1], out["k"][1],
                     out["v"][1], inp.cu_seqlens, inp.scale, dict(inp.meta))


def make_fp8_config(name: str) -> Fp8Inputs:
    """The FP8 version of a named workload (same seeds and structure, quantised per tensor)."""
    return quantize_fp8(make_config(name), name + "_fp8")
