"""The C-ABI library: it loads, exports every declared symbol, and validates arguments on the
host before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import long_sequence_video_amd as lsv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsv_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(lsv.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lsv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


GEN_HEADER = os.path.join(ROOT, "include", "lsvgen.h")


def test_generator_library_exports_every_declared_symbol():
    from long_sequence_video_amd import inputs as gen
    text = re.sub(r"/\*.*?\*/", "", open(GEN_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(lsvgen_\w+)\s*\(", text)))
    assert names == ["lsvgen_amax_bf16", "lsvgen_choose", "lsvgen_normal_bf16", "lsvgen_normal_f64_at",
                     "lsvgen_quantize_e4m3_bf16", "lsvgen_rms_normalize_bf16", "lsvgen_scale_rows_bf16"]
    lib = ctypes.CDLL(gen.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_generator_rejects_bad_arguments():
    from long_sequence_video_amd import inputs as gen
    lib = ctypes.CDLL(gen.LIB_PATH)
    assert lib.lsvgen_normal_bf16(None, ctypes.c_int64(-1), ctypes.c_uint64(1), ctypes.c_uint32(0)) == -1
    assert lib.lsvgen_normal_bf16(None, ctypes.c_int64(4), ctypes.c_uint64(1), ctypes.c_uint32(0)) == -1
    assert lib.lsvgen_normal_bf16(None, ctypes.c_int64(0), ctypes.c_uint64(1), ctypes.c_uint32(0)) == 0
    assert lib.lsvgen_choose(None, ctypes.c_int64(3), ctypes.c_int64(2), None, ctypes.c_uint64(1),
                             ctypes.c_uint32(3)) == -1
    u8 = (ctypes.c_uint8 * 4)()
    u16 = (ctypes.c_uint16 * 4)()
    assert lib.lsvgen_quantize_e4m3_bf16(u16, ctypes.c_int64(4), ctypes.c_double(0.0), u8) == -1
    assert lib.lsvgen_quantize_e4m3_bf16(u16, ctypes.c_int64(4), ctypes.c_double(float("nan")), u8) == -1
    assert lib.lsvgen_quantize_e4m3_bf16(None, ctypes.c_int64(4), ctypes.c_double(1.0), u8) == -1
    assert lib.lsvgen_quantize_e4m3_bf16(u16, ctypes.c_int64(-1), ctypes.c_double(1.0), u8) == -1
    assert lib.lsvgen_amax_bf16(u16, ctypes.c_int64(4), None) == -1


def test_status_strings():
    assert lsv.lsv_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert lsv.lsv_status_string(code) not in ("ok", "unknown status")
    assert lsv.lsv_status_string(-99) == "unknown status"


def test_tile_config():
    bq, bk = lsv.lsv_tile_config()
    assert bq > 0 and bk > 0 and bq % 32 == 0 and bk % 32 == 0


# Fake, suitably aligned addresses: validation must reject before touching them.
A = 1 << 20


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(head_dim=8), lsv.LSV_ERR_UNSUPPORTED),          # the pages' q [7, 2, 8] example
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_seqs=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(max_seqlen=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(total_tokens=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=-0.1), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=float("inf")), lsv.LSV_ERR_INVALID_ARG),
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(lse=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(cu=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(v=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(o=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(lse=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(total_tokens=1 << 31), lsv.LSV_ERR_UNSUPPORTED),
    # one head's K/V rows of a segment must be addressable with 32-bit byte offsets
    (dict(max_seqlen=299_594, total_tokens=299_594, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),
    # successful no-ops: nothing to compute, nothing launched
    (dict(n_seqs=0), lsv.LSV_OK),
    (dict(max_seqlen=0), lsv.LSV_OK),
    (dict(total_tokens=0), lsv.LSV_OK),
    (dict(n_seqs=0, q=0, k=0, v=0, o=0, lse=0, cu=0), lsv.LSV_OK),
])
def test_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, n_seqs=1, max_seqlen=10, total_tokens=10, n_heads=4, head_dim=128,
             scale=0.125)
    a.update(args)
    rc = lsv.lsv_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["n_seqs"], a["max_seqlen"],
                          a["total_tokens"], a["n_heads"], a["head_dim"], a["scale"], None)
    assert rc == code


def test_flops_count():
    assert lsv.flops([19394, 38000, 104000], 56) == 4 * (19394 ** 2 + 38000 ** 2 + 104000 ** 2) * 56 * 128
    assert lsv.flops([104000], 56) == 4 * 104000 ** 2 * 56 * 128


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(rotary_dim=40), lsv.LSV_ERR_UNSUPPORTED),       # not a multiple of 16
    (dict(rotary_dim=144), lsv.LSV_ERR_UNSUPPORTED),      # wider than the head
    (dict(rotary_dim=-16), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(batch=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(seq_len=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(eps=-1e-5), lsv.LSV_ERR_INVALID_ARG),
    (dict(eps=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(eps=float("inf")), lsv.LSV_ERR_INVALID_ARG),
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(k_weight=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(out=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(cos=0), lsv.LSV_ERR_INVALID_ARG),               # tables are needed when rotary_dim > 0
    (dict(k=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(sin=A + 4), lsv.LSV_ERR_ALIGNMENT),
    (dict(q_weight=A + 1), lsv.LSV_ERR_ALIGNMENT),
    (dict(batch=4, seq_len=40000, n_heads=14000), lsv.LSV_ERR_UNSUPPORTED),  # 2^31 rows or more
    (dict(batch=1 << 40, seq_len=1 << 40), lsv.LSV_ERR_UNSUPPORTED),          # no overflow in the check
    # successful no-ops
    (dict(batch=0), lsv.LSV_OK),
    (dict(seq_len=0, q=0, k=0, v=0, out=0), lsv.LSV_OK),
])
def test_prologue_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, q_weight=A, k_weight=A, cos=A, sin=A, out=A, batch=1, seq_len=10, n_heads=4,
             head_dim=128, rotary_dim=96, eps=1e-5)
    a.update(args)
    rc = lsv.lsv_qkv_prologue(a["q"], a["k"], a["v"], a["q_weight"], a["k_weight"], a["cos"], a["sin"], a["out"],
                              a["batch"], a["seq_len"], a["n_heads"], a["head_dim"], a["rotary_dim"], a["eps"], None)
    assert rc == code


def test_bwd_workspace_size():
    assert lsv.lsv_attn_bwd_workspace_size(161394, 56) == 8 * 161394 * 56
    assert lsv.lsv_attn_bwd_workspace_size(0, 4) == 0
    assert lsv.lsv_attn_bwd_workspace_size(-1, 4) == -1
    assert lsv.lsv_attn_bwd_workspace_size(10, 0) == -1


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_seqs=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(o=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dout=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dk=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws_bytes=8 * 10 * 4 - 1), lsv.LSV_ERR_INVALID_ARG),   # one byte short
    (dict(dv=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(dout=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(ws=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(total_tokens=1 << 31, ws_bytes=1 << 40), lsv.LSV_ERR_UNSUPPORTED),
    (dict(total_tokens=40_000_000, n_heads=56, ws_bytes=1 << 40), lsv.LSV_ERR_UNSUPPORTED),  # T*H >= 2^31
    (dict(max_seqlen=299_594, total_tokens=299_594, n_heads=56, ws_bytes=1 << 40), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_seqs=0), lsv.LSV_OK),
    (dict(max_seqlen=0, ws=0), lsv.LSV_OK),
])
def test_bwd_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, cu=A, n_seqs=1, max_seqlen=10, total_tokens=10,
             n_heads=4, head_dim=128, scale=0.125, ws=A, ws_bytes=8 * 10 * 4)
    a.update(args)
    rc = lsv.lsv_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["cu"],
                          a["n_seqs"], a["max_seqlen"], a["total_tokens"], a["n_heads"], a["head_dim"], a["scale"],
                          a["ws"], a["ws_bytes"], None)
    assert rc == code


def test_bwd_noalloc_max_rows():
    """The no-alloc backward's scratch holds two fp32 values for 2^24 (token, head) rows: one
    segment of 299,593 tokens at 56 heads, the largest the 32-bit offsets allow, fits."""
    assert lsv.lsv_attn_bwd_noalloc_max_rows() == 1 << 24
    assert 299_593 * 56 <= lsv.lsv_attn_bwd_noalloc_max_rows()


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_seqs=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=float("inf")), lsv.LSV_ERR_INVALID_ARG),
    (dict(o=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dq=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dv=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(lse=A + 2), lsv.LSV_ERR_ALIGNMENT),
    # beyond the scratch: one (token, head) row more than 2^24
    (dict(total_tokens=(1 << 24) + 1, n_heads=1, max_seqlen=10), lsv.LSV_ERR_UNSUPPORTED),
    (dict(total_tokens=299_594, n_heads=56, max_seqlen=10), lsv.LSV_ERR_UNSUPPORTED),
    (dict(max_seqlen=299_594, total_tokens=299_594, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_seqs=0), lsv.LSV_OK),
    (dict(max_seqlen=0), lsv.LSV_OK),
    (dict(total_tokens=0), lsv.LSV_OK),
])
def test_bwd_noalloc_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, cu=A, n_seqs=1, max_seqlen=10, total_tokens=10,
             n_heads=4, head_dim=128, scale=0.125)
    a.update(args)
    rc = lsv.lsv_attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                                  a["cu"], a["n_seqs"], a["max_seqlen"], a["total_tokens"], a["n_heads"],
                                  a["head_dim"], a["scale"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dq=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dk=-1.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dv=float("inf")), lsv.LSV_ERR_INVALID_ARG),
    (dict(dq=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(dq=1e30, dk=1e30), lsv.LSV_ERR_INVALID_ARG),     # scale * dq * dk overflows fp32
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(k=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(lse=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(max_seqlen=599_187, total_tokens=599_187, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),  # 32-bit offsets
    (dict(n_seqs=0), lsv.LSV_OK),
    (dict(total_tokens=0), lsv.LSV_OK),
])
def test_fp8_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, dq=0.01, dk=0.01, dv=0.01, n_seqs=1, max_seqlen=10, total_tokens=10,
             n_heads=4, head_dim=128, scale=0.125)
    a.update(args)
    rc = lsv.lsv_attn_fwd_fp8(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"], a["lse"], a["cu"],
                              a["n_seqs"], a["max_seqlen"], a["total_tokens"], a["n_heads"], a["head_dim"],
                              a["scale"], None)
    assert rc == code


def test_split_workspace_size():
    assert lsv.lsv_attn_fwd_split_workspace_size(19394, 14, 3) == 3 * 19394 * 14 * 129 * 4
    assert lsv.lsv_attn_fwd_split_workspace_size(10, 2, 1) == 0
    assert lsv.lsv_attn_fwd_split_workspace_size(0, 2, 2) == 0
    for bad in ((10, 2, 0), (10, 2, 9), (10, 0, 2), (-1, 2, 2)):
        assert lsv.lsv_attn_fwd_split_workspace_size(*bad) == -1


@pytest.mark.parametrize("args,code", [
    (dict(n_split=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_split=9), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_split=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(ws_bytes=2 * 10 * 4 * 129 * 4 - 1), lsv.LSV_ERR_INVALID_ARG),   # one byte short
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(o=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(max_seqlen=299_594, total_tokens=299_594, n_heads=56, ws_bytes=1 << 42), lsv.LSV_ERR_UNSUPPORTED),
    # successful no-ops, with any split and without a workspace
    (dict(n_seqs=0, ws=0), lsv.LSV_OK),
    (dict(max_seqlen=0, ws=0), lsv.LSV_OK),
    (dict(n_split=1, n_seqs=0, ws=0), lsv.LSV_OK),
])
def test_split_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, n_seqs=1, max_seqlen=10, total_tokens=10, n_heads=4, head_dim=128,
             scale=0.125, n_split=2, ws=A, ws_bytes=2 * 10 * 4 * 129 * 4)
    a.update(args)
    rc = lsv.lsv_attn_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["n_seqs"], a["max_seqlen"],
                                a["total_tokens"], a["n_heads"], a["head_dim"], a["scale"], a["n_split"], a["ws"],
                                a["ws_bytes"], None)
    assert rc == code


def test_choose_split():
    """Host-side choice of the key split: only long segments in launches that leave the last
    round of 256 compute units mostly idle are split."""
    assert lsv.choose_split([19394], 14) == 2      # 1,064 workgroups (4.16 rounds) -> 2,128 (8.31)
    assert lsv.choose_split([4096], 56) == 1       # ranges would hold under 8,192 keys
    assert lsv.choose_split([19394, 38000, 104000], 56) == 1   # 35,392 workgroups: 99% full
    assert lsv.choose_split([104000], 56) == 1
    assert lsv.choose_split([38000], 56) == 1
    assert lsv.choose_split([], 4) == 1 and lsv.choose_split([0, 0], 4) == 1
    assert lsv.choose_split([19394], 14, min_range_keys=1024) == 4   # fullest rounds: 16.6 of 17


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(rotary_dim=8), lsv.LSV_ERR_UNSUPPORTED),
    (dict(rotary_dim=144), lsv.LSV_ERR_UNSUPPORTED),
    (dict(rotary_dim=-16), lsv.LSV_ERR_UNSUPPORTED),
    (dict(eps=-1.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(eps=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(scale=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(w=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(cos=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(w=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(sin=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(o=A + 2), lsv.LSV_ERR_ALIGNMENT),
    (dict(max_seqlen=299_594, total_tokens=299_594, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),
    (dict(n_seqs=0), lsv.LSV_OK),
    (dict(rotary_dim=0, cos=0, sin=0, n_seqs=0), lsv.LSV_OK),
])
def test_attn_fwd_qnorm_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, w=A, cos=A, sin=A, rotary_dim=96, eps=1e-5, o=A, lse=A, cu=A, n_seqs=1, max_seqlen=10,
             total_tokens=10, n_heads=4, head_dim=128, scale=0.125)
    a.update(args)
    rc = lsv.lsv_attn_fwd_qnorm(a["q"], a["k"], a["v"], a["w"], a["cos"], a["sin"], a["rotary_dim"], a["eps"], a["o"],
                                a["lse"], a["cu"], a["n_seqs"], a["max_seqlen"], a["total_tokens"], a["n_heads"],
                                a["head_dim"], a["scale"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(rotary_dim=24), lsv.LSV_ERR_UNSUPPORTED),
    (dict(eps=float("inf")), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_heads=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(total_tokens=-1), lsv.LSV_ERR_INVALID_ARG),
    (dict(x=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(w=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(sin=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(out=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(w=A + 1), lsv.LSV_ERR_ALIGNMENT),
    (dict(total_tokens=1 << 31), lsv.LSV_ERR_UNSUPPORTED),
    (dict(total_tokens=40_000_000, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),   # rows >= 2^31
    (dict(total_tokens=0), lsv.LSV_OK),
    (dict(rotary_dim=0, cos=0, sin=0, total_tokens=0), lsv.LSV_OK),
])
def test_norm_rope_validation_before_any_hip_call(args, code):
    a = dict(x=A, w=A, cos=A, sin=A, out=A, total_tokens=10, n_heads=4, head_dim=128, rotary_dim=96, eps=1e-5)
    a.update(args)
    rc = lsv.lsv_norm_rope(a["x"], a["w"], a["cos"], a["sin"], a["out"], a["total_tokens"], a["n_heads"],
                           a["head_dim"], a["rotary_dim"], a["eps"], None)
    assert rc == code


def test_tail_plans():
    """lsv_attn_fwd_tail's plans (host arithmetic): per XCD, ceil(n / 8) tiles, the ones past its
    last whole round of compute_units / 8 cut when they are at most a quarter of it."""
    assert lsv.lsv_attn_fwd_tail_plan(1, 19394, 14, 256) == (6, 40)      # 1,064 tiles: 133 per XCD, 5 past
    assert lsv.lsv_attn_fwd_tail_plan(3, 104000, 56, 256) == (8, 24)     # the 161,394-token pack: 3 past
    assert lsv.lsv_attn_fwd_tail_plan(1, 104000, 56, 256) == (8, 8)      # 2,849 per XCD: 1 past
    assert lsv.lsv_attn_fwd_tail_plan(1, 4096, 56, 256) == (1, 0)        # 112 per XCD: half a round left whole
    assert lsv.lsv_attn_fwd_tail_plan(1, 38000, 56, 256) == (1, 0)       # 1,043 per XCD: 19 past, over a quarter
    assert lsv.lsv_attn_fwd_tail_plan(1, 256, 4, 256) == (1, 0)          # 4 tiles: ranges would be under 1,024 keys
    assert lsv.lsv_attn_fwd_tail_plan(1, 5000, 1, 16) == (1, 0)          # 20 tiles, 3 per XCD on 2 slots: half a round
    # n not a multiple of 8 (the sp=4 shares of the 38,000- and 104,000-token clips at 14 heads)
    assert lsv.lsv_attn_fwd_tail_plan(1, 38000, 14, 256) == (6, 40)      # 2,086 tiles: 261 per XCD, 5 past
    assert lsv.lsv_attn_fwd_tail_plan(1, 104000, 14, 256) == (1, 0)      # 5,698 tiles: 713 per XCD, 9 past
    assert lsv.lsv_attn_fwd_tail_plan(1, 5000, 7, 128) == (4, 16)        # 140 tiles: 18 per XCD, 2 past
    assert lsv.lsv_attn_fwd_tail_plan(1, 1024, 8, 256) == (1, 0)         # ranges would be under 1,024 keys
    assert lsv.lsv_attn_fwd_tail_plan(2, 5000, 1, 256) == (4, 40)        # every tile cut: 5 per XCD of 32 slots
    assert lsv.lsv_attn_fwd_tail_plan(2, 9000, 4, 256) == (8, 32)
    with pytest.raises(lsv.LsvError):
        lsv.lsv_attn_fwd_tail_plan(1, 4096, 56, 100)                    # not a multiple of 8
    assert lsv.lsv_attn_fwd_tail_workspace_size(256) == 256 * 256 * 129 * 4
    assert lsv.lsv_attn_fwd_tail_workspace_size(12) == -1


@pytest.mark.parametrize("args,code", [
    (dict(units=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(units=100), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=0), lsv.LSV_ERR_INVALID_ARG),             # this plan cuts 6 ranges: a workspace is needed
    (dict(ws=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(ws_bytes=40 * 6 * 256 * 129 * 4 - 1), lsv.LSV_ERR_INVALID_ARG),
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(n_seqs=0, ws=0), lsv.LSV_OK),
])
def test_tail_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, n_seqs=1, max_seqlen=19394, total_tokens=19394, n_heads=14,
             head_dim=128, scale=0.125, units=256, ws=A, ws_bytes=40 * 6 * 256 * 129 * 4)
    a.update(args)
    rc = lsv.lsv_attn_fwd_tail(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["n_seqs"], a["max_seqlen"],
                               a["total_tokens"], a["n_heads"], a["head_dim"], a["scale"], a["units"], a["ws"],
                               a["ws_bytes"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(units=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(units=100), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=0), lsv.LSV_ERR_INVALID_ARG),             # this plan cuts 6 ranges: a workspace is needed
    (dict(ws=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(ws_bytes=40 * 6 * 256 * 129 * 4 - 1), lsv.LSV_ERR_INVALID_ARG),
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(dq=0.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(dv=float("nan")), lsv.LSV_ERR_INVALID_ARG),
    (dict(dq=1e30, dk=1e30), lsv.LSV_ERR_INVALID_ARG),     # scale * dq * dk overflows fp32
    (dict(q=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(k=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(max_seqlen=599_187, total_tokens=599_187, n_heads=56), lsv.LSV_ERR_UNSUPPORTED),  # 32-bit offsets
    (dict(n_seqs=0, ws=0), lsv.LSV_OK),
])
def test_fp8_tail_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cu=A, dq=0.01, dk=0.01, dv=0.01, n_seqs=1, max_seqlen=19394,
             total_tokens=19394, n_heads=14, head_dim=128, scale=0.125, units=256, ws=A,
             ws_bytes=40 * 6 * 256 * 129 * 4)
    a.update(args)
    rc = lsv.lsv_attn_fwd_fp8_tail(a["q"], a["k"], a["v"], a["dq"], a["dk"], a["dv"], a["o"], a["lse"], a["cu"],
                                   a["n_seqs"], a["max_seqlen"], a["total_tokens"], a["n_heads"], a["head_dim"],
                                   a["scale"], a["units"], a["ws"], a["ws_bytes"], None)
    assert rc == code


@pytest.mark.parametrize("args,code", [
    (dict(units=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(units=100), lsv.LSV_ERR_INVALID_ARG),
    (dict(ws=0), lsv.LSV_ERR_INVALID_ARG),             # this plan cuts 6 ranges: a workspace is needed
    (dict(ws=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(ws_bytes=40 * 6 * 256 * 129 * 4 - 1), lsv.LSV_ERR_INVALID_ARG),
    (dict(rotary_dim=8), lsv.LSV_ERR_UNSUPPORTED),
    (dict(eps=-1.0), lsv.LSV_ERR_INVALID_ARG),
    (dict(head_dim=64), lsv.LSV_ERR_UNSUPPORTED),
    (dict(w=0), lsv.LSV_ERR_INVALID_ARG),
    (dict(sin=A + 8), lsv.LSV_ERR_ALIGNMENT),
    (dict(n_seqs=0, ws=0), lsv.LSV_OK),
])
def test_attn_fwd_qnorm_tail_validation_before_any_hip_call(args, code):
    a = dict(q=A, k=A, v=A, w=A, cos=A, sin=A, rotary_dim=96, eps=1e-5, o=A, lse=A, cu=A, n_seqs=1,
             max_seqlen=19394, total_tokens=19394, n_heads=14, head_dim=128, scale=0.125, units=256, ws=A,
             ws_bytes=40 * 6 * 256 * 129 * 4)
    a.update(args)
    rc = lsv.lsv_attn_fwd_qnorm_tail(a["q"], a["k"], a["v"], a["w"], a["cos"], a["sin"], a["rotary_dim"], a["eps"],
                                     a["o"], a["lse"], a["cu"], a["n_seqs"], a["max_seqlen"], a["total_tokens"],
                                     a["n_heads"], a["head_dim"], a["scale"], a["units"], a["ws"], a["ws_bytes"],
                                     None)
    assert rc == code


def test_library_shares_torchs_hip_runtime():
    """Loading the library before torch is imported must not map a second HIP runtime: torch ships
    its own, and kernels registered with one runtime cannot run on the other's streams or memory
    (a fresh process, so nothing has imported torch yet)."""
    import subprocess
    import sys
    code = ("import long_sequence_video_amd as lsv\n"
            "lsv.load_library()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_tail_plan_invariants_over_random_sizes():
    """lsv_attn_fwd_tail_plan against the contract its header states, on 3,000 seeded random sizes:
    with n tiles and P = ceil(n / 8) per XCD of units / 8 slots, the cut tiles are the t = P mod
    slots past the last whole round, cut only when 1 <= t <= slots / 4, into at most 8 ranges,
    at most slots / t (so each XCD's pieces fill at most one round) and at most max_seqlen / 1024
    (ranges of >= 1024 keys); the pieces fit the workspace lsv_attn_fwd_tail_workspace_size
    promises; nothing is cut otherwise."""
    import numpy as np
    rng = np.random.default_rng(2024)
    for _ in range(3000):
        n_seqs = int(rng.integers(1, 6))
        max_seqlen = int(rng.choice([rng.integers(1, 4096), rng.integers(4096, 300_000)]))
        heads = int(rng.integers(1, 65))
        units = 8 * int(rng.integers(1, 41))
        split, n_tail = lsv.lsv_attn_fwd_tail_plan(n_seqs, max_seqlen, heads, units)
        n = -(-max_seqlen // 256) * n_seqs * heads
        slots, t = units // 8, -(-n // 8) % (units // 8)
        if split == 1:
            assert n_tail == 0
            assert t == 0 or t > slots // 4 or min(8, slots // t, max_seqlen // 1024) < 2
            continue
        assert n_tail == 8 * t and 1 <= t <= slots // 4
        assert 2 <= split <= min(8, slots // t, max_seqlen // 1024)
        assert split == min(8, slots // t, max_seqlen // 1024)
        assert t * split <= slots
        assert n_tail * split * 256 * 129 * 4 <= lsv.lsv_attn_fwd_tail_workspace_size(units)
