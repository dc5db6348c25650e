"""Boundary contract (CPU only): the library loads, exports what include/fa_fwd.h declares,
and rejects every invalid argument on the host before any HIP call. The strict-backend
rule comes from "h3-blackwell-runtime/FLASH4.md", section "API": matching FP16/BF16
tensors, matching shapes, a supported head dim, and an error instead of a kernel change.
"""

import ctypes
import math

import pytest
import torch

import exact_attention_06_amd as fa
from exact_attention_06_amd import _lib

A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced by the checks
GOOD = dict(q=A, k=A + 0x100, v=A + 0x200, o=A + 0x300, lse=A + 0x400, B=2, Nq=300, Nk=300,
            Hq=8, Hkv=2, d=128, causal=0, scale=0.0884)


def _check(**kw):
    a = dict(GOOD, **kw)
    return fa.check_args(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"], a["Nk"], a["Hq"],
                         a["Hkv"], a["d"], a["causal"], a["scale"])


def _fwd(fn, **kw):
    a = dict(GOOD, **kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"], a["Nk"], a["Hq"], a["Hkv"],
              a["d"], a["causal"], ctypes.c_float(a["scale"]), None)


def test_library_exports_every_header_symbol():
    lib = _lib.load()
    names = _lib.header_symbols()
    assert set(names) == {"fa_fwd", "fa_fwd_f16", "fa_strerror", "fa_fwd_check", "fa_bwd", "fa_bwd_f16",
                          "fa_bwd_workspace_bytes", "fa_fwd_varlen", "fa_fwd_varlen_f16", "fa_fwd_paged",
                          "fa_fwd_paged_f16", "fa_fwd_splitkv", "fa_fwd_splitkv_f16",
                          "fa_fwd_splitkv_workspace_bytes", "fa_fwd_num_splits", "fa_fwd_fp8",
                          "fa_fwd_var_splitkv_workspace_bytes", "fa_fwd_varlen_splitkv",
                          "fa_fwd_varlen_splitkv_f16", "fa_fwd_paged_splitkv", "fa_fwd_paged_splitkv_f16",
                          "fa_fwd_var_num_splits", "fa_bwd_noalloc", "fa_set_grid_order"}
    for n in names:
        assert hasattr(lib, n), n


def test_valid_arguments_pass():
    assert _check() == _lib.FA_OK
    assert _check(d=256, causal=1, Hkv=8) == _lib.FA_OK
    assert _check(Nq=1, Nk=1) == _lib.FA_OK
    assert _check(Nq=5, Nk=9000) == _lib.FA_OK
    assert _check(scale=0.0) == _lib.FA_OK
    # a negative scale is a valid softmax(scale * Q K^T) (scores of the opposite sign)
    assert _check(scale=-0.0884) == _lib.FA_OK
    assert _check(scale=-1e30) == _lib.FA_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointer(field):
    assert _check(**{field: 0}) == _lib.FA_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(Nk=-1), dict(Hq=0), dict(Hkv=0),
                                dict(Hq=8, Hkv=3), dict(Hq=2, Hkv=4)])
def test_bad_shape(kw):
    assert _check(**kw) == _lib.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, 64, 96, 127, 192, 384, 1024])
def test_bad_head_dim(d):
    assert _check(d=d) == _lib.FA_ERR_HEADDIM


def test_head_dim_512_only_for_the_dense_forward():
    # d = 512 runs on the dense forward kernel only; every other entry point rejects it
    assert _check(d=512) == _lib.FA_OK
    assert _check(d=512, causal=1, Hkv=8) == _lib.FA_OK
    lib = _lib.load()
    assert _bwd(lib.fa_bwd, d=512) == _lib.FA_ERR_HEADDIM
    assert _varlen(lib.fa_fwd_varlen, d=512) == _lib.FA_ERR_HEADDIM
    assert _paged(lib.fa_fwd_paged, d=512) == _lib.FA_ERR_HEADDIM
    assert _split(lib.fa_fwd_splitkv, d=512) == _lib.FA_ERR_HEADDIM
    assert _fp8(d=512) == _lib.FA_ERR_HEADDIM
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 300, 8, 512, 2) == 0
    assert lib.fa_fwd_num_splits(1, 1024, 1024, 8, 512, 0) == 1


def test_causal_needs_square():
    assert _check(causal=1, Nq=300, Nk=301) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _check(causal=0, Nq=300, Nk=301) == _lib.FA_OK


@pytest.mark.parametrize("s", [math.inf, -math.inf, math.nan, -math.nan])
def test_bad_scale(s):
    assert _check(scale=s) == _lib.FA_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(q=A + 8), dict(k=A + 2), dict(v=A + 4), dict(o=A + 1), dict(lse=A + 2)])
def test_misaligned(kw):
    assert _check(**kw) == _lib.FA_ERR_ALIGN


def test_lse_4_byte_alignment_is_enough():
    assert _check(lse=A + 4) == _lib.FA_OK


def test_too_large_grid():
    assert _check(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 12, Nk=1 << 12) == _lib.FA_ERR_TOO_LARGE


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f16"])
def test_entry_points_reject_before_any_hip_call(entry):
    # These calls must return on the host; with no GPU present a HIP call would fail differently.
    fn = getattr(_lib.load(), entry)
    assert _fwd(fn, q=0) == _lib.FA_ERR_NULL
    assert _fwd(fn, d=64) == _lib.FA_ERR_HEADDIM
    assert _fwd(fn, causal=1, Nk=17) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _fwd(fn, Hkv=3) == _lib.FA_ERR_SHAPE
    assert _fwd(fn, scale=math.nan) == _lib.FA_ERR_SCALE
    assert _fwd(fn, o=A + 2) == _lib.FA_ERR_ALIGN


def test_strerror_covers_codes():
    seen = set()
    for code in range(-11, 1):
        msg = _lib.strerror(code)
        assert msg and msg != "unknown fa status code"
        seen.add(msg)
    assert len(seen) == 12
    assert _lib.strerror(-99) == "unknown fa status code"


def test_python_layer_rejects_cpu_tensors():
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q)


def test_python_layer_error_type():
    err = fa.FaError(_lib.FA_ERR_HEADDIM, _lib.strerror(_lib.FA_ERR_HEADDIM))
    assert isinstance(err, ValueError) and "head dim" in str(err)


def _bwd(fn, **kw):
    a = dict(GOOD, **kw)
    ws = a.get("ws", A + 0x800)
    wsb = a.get("wsb", 4 * a["B"] * a["Hq"] * a["Nq"])
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a.get("do", A + 0x500), a.get("dq", A + 0x600),
              a.get("dk", A + 0x700), a.get("dv", A + 0x780), ws, wsb, a["B"], a["Nq"], a["Nk"], a["Hq"],
              a["Hkv"], a["d"], a["causal"], ctypes.c_float(a["scale"]), None)


def test_bwd_workspace_size():
    lib = _lib.load()
    assert lib.fa_bwd_workspace_bytes(2, 300, 8) == 4 * 2 * 300 * 8
    assert lib.fa_bwd_workspace_bytes(0, 300, 8) == 0


@pytest.mark.parametrize("entry", ["fa_bwd", "fa_bwd_f16"])
def test_bwd_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    assert _bwd(fn, q=0) == _lib.FA_ERR_NULL
    assert _bwd(fn, do=0) == _lib.FA_ERR_NULL
    assert _bwd(fn, dk=0) == _lib.FA_ERR_NULL
    assert _bwd(fn, d=96) == _lib.FA_ERR_HEADDIM
    assert _bwd(fn, causal=1, Nk=17) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _bwd(fn, dq=A + 0x604) == _lib.FA_ERR_ALIGN
    assert _bwd(fn, ws=0) == _lib.FA_ERR_WORKSPACE
    assert _bwd(fn, wsb=4 * 2 * 300 * 8 - 4) == _lib.FA_ERR_WORKSPACE
    assert _bwd(fn, ws=A + 0x802) == _lib.FA_ERR_WORKSPACE


def _bwd_noalloc(**kw):
    a = dict(GOOD, **kw)
    return _lib.load().fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a.get("do", A + 0x500),
                                      a.get("dq", A + 0x600), a.get("dk", A + 0x700), a.get("dv", A + 0x780),
                                      a["B"], a["Nq"], a["Nk"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                      ctypes.c_float(a["scale"]), None)


def test_bwd_noalloc_rejects_before_any_hip_call():
    # the allocation-free backward pass checks as fa_bwd does, then its fixed scratch limit
    assert _bwd_noalloc(q=0) == _lib.FA_ERR_NULL
    assert _bwd_noalloc(do=0) == _lib.FA_ERR_NULL
    assert _bwd_noalloc(dv=0) == _lib.FA_ERR_NULL
    assert _bwd_noalloc(d=96) == _lib.FA_ERR_HEADDIM
    assert _bwd_noalloc(d=512) == _lib.FA_ERR_HEADDIM
    assert _bwd_noalloc(causal=1, Nk=17) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _bwd_noalloc(Hkv=3) == _lib.FA_ERR_SHAPE
    assert _bwd_noalloc(scale=math.nan) == _lib.FA_ERR_SCALE
    assert _bwd_noalloc(dq=A + 0x604) == _lib.FA_ERR_ALIGN
    assert _bwd_noalloc(do=A + 0x508) == _lib.FA_ERR_ALIGN
    rows = _lib.FA_BWD_NOALLOC_MAX_ROWS
    assert _bwd_noalloc(B=1, Hq=16, Hkv=16, Nq=rows // 16 + 1, Nk=4096) == _lib.FA_ERR_SCRATCH
    assert _bwd_noalloc(B=2, Hq=8, Hkv=8, Nq=rows // 16 + 1, Nk=rows // 16 + 1, causal=1) == _lib.FA_ERR_SCRATCH
    assert "scratch" in _lib.strerror(_lib.FA_ERR_SCRATCH)


# ---- variable-length and paged entry points: every rejection happens on the host

VGOOD = dict(q=A, k=A + 0x100, v=A + 0x200, o=A + 0x300, lse=A + 0x400, cu_q=A + 0x500, cu_k=A + 0x600,
             used=A + 0x700, bt=A + 0x800, B=3, max_q=64, total_q=100, total_k=200, num_pages=10,
             page_size=128, max_pages=4, Hq=8, Hkv=2, d=128, causal=1, scale=0.0884)


def _varlen(fn, **kw):
    a = dict(VGOOD, **kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"], a["cu_k"], a["used"], a["B"], a["max_q"],
              a["total_q"], a["total_k"], a["Hq"], a["Hkv"], a["d"], a["causal"], ctypes.c_float(a["scale"]), None)


def _paged(fn, **kw):
    a = dict(VGOOD, **kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu_q"], a["used"], a["bt"], a["B"], a["max_q"],
              a["total_q"], a["num_pages"], a["page_size"], a["max_pages"], a["Hq"], a["Hkv"], a["d"],
              a["causal"], ctypes.c_float(a["scale"]), None)


@pytest.mark.parametrize("entry", ["fa_fwd_varlen", "fa_fwd_varlen_f16"])
def test_varlen_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    for f in ("q", "k", "v", "o", "lse", "cu_q", "cu_k"):
        assert _varlen(fn, **{f: 0}) == _lib.FA_ERR_NULL, f
    for kw in (dict(B=0), dict(max_q=0), dict(total_q=0), dict(total_k=-1), dict(Hq=0), dict(Hkv=3)):
        assert _varlen(fn, **kw) == _lib.FA_ERR_SHAPE, kw
    assert _varlen(fn, d=192) == _lib.FA_ERR_HEADDIM
    assert _varlen(fn, scale=math.inf) == _lib.FA_ERR_SCALE
    for kw in (dict(q=A + 8), dict(o=A + 4), dict(lse=A + 2), dict(cu_q=A + 1), dict(cu_k=A + 2),
               dict(used=A + 3)):
        assert _varlen(fn, **kw) == _lib.FA_ERR_ALIGN, kw
    assert _varlen(fn, B=1 << 20, Hq=1 << 10, Hkv=1 << 10, max_q=1 << 12) == _lib.FA_ERR_TOO_LARGE


@pytest.mark.parametrize("entry", ["fa_fwd_paged", "fa_fwd_paged_f16"])
def test_paged_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    for f in ("q", "k", "v", "o", "lse", "cu_q", "used", "bt"):
        assert _paged(fn, **{f: 0}) == _lib.FA_ERR_NULL, f
    for kw in (dict(B=0), dict(max_q=0), dict(total_q=0), dict(Hq=4, Hkv=8)):
        assert _paged(fn, **kw) == _lib.FA_ERR_SHAPE, kw
    for kw in (dict(page_size=0), dict(page_size=96), dict(page_size=-128), dict(num_pages=0),
               dict(max_pages=0), dict(max_pages=1 << 24), dict(num_pages=1 << 24)):
        assert _paged(fn, **kw) == _lib.FA_ERR_PAGE, kw
    assert _paged(fn, d=64) == _lib.FA_ERR_HEADDIM
    assert _paged(fn, scale=-math.inf) == _lib.FA_ERR_SCALE
    for kw in (dict(k=A + 8), dict(bt=A + 2), dict(used=A + 1)):
        assert _paged(fn, **kw) == _lib.FA_ERR_ALIGN, kw


def test_varlen_python_layer_rejects_cpu_tensors():
    q = torch.zeros(10, 2, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_varlen(q, q, q, cu, cu, 10)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_paged(q, q[None], q[None], cu, cu[1:], cu[None], 10)


# ---- split-KV entry points

def _split(fn, **kw):
    a = dict(GOOD, **kw)
    splits = a.get("splits", 4)
    ws = a.get("ws", A + 0x1000)
    wsb = a.get("wsb", splits * a["B"] * a["Hq"] * a["Nq"] * (a["d"] + 1) * 4)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], ws, wsb, a["B"], a["Nq"], a["Nk"], a["Hq"], a["Hkv"],
              a["d"], a["causal"], ctypes.c_float(a["scale"]), splits, None)


def test_splitkv_workspace_size():
    lib = _lib.load()
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 300, 8, 128, 3) == 3 * 2 * 8 * 300 * 129 * 4
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 300, 8, 256, 1) == 2 * 8 * 300 * 257 * 4
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 300, 8, 64, 3) == 0
    assert lib.fa_fwd_splitkv_workspace_bytes(2, 300, 8, 128, 0) == 0


def test_num_splits_choice():
    # a grid that fills the GPU is not split; few heads and short sequences are (the measured
    # rule table of fa_fwd.hip)
    assert fa.num_splits(4, 8192, 8192, 8, 256) == 1
    assert fa.num_splits(32, 1024, 1024, 8, 256) == 1
    assert fa.num_splits(1, 100, 100, 8, 256) == 1                   # too few key tiles to split
    assert fa.num_splits(1, 1024, 1024, 8, 256) == 3                 # 64 workgroups, 32 key tiles
    assert fa.num_splits(1, 1024, 1024, 8, 256, causal=True) == 4
    assert fa.num_splits(2, 1024, 1024, 8, 256) == 1                 # 128 workgroups, 32 key tiles
    assert fa.num_splits(2, 1024, 1024, 8, 256, causal=True) == 2    # 128 workgroups, causal
    assert fa.num_splits(1, 2048, 2048, 8, 256) == 3                 # 128 workgroups, 64 key tiles
    assert fa.num_splits(1, 2048, 2048, 8, 256, causal=True) == 2
    assert fa.num_splits(1, 4096, 4096, 8, 256) == 1
    assert fa.num_splits(1, 4096, 4096, 8, 256, causal=True) == 3    # 256 workgroups, 128 key tiles
    assert fa.num_splits(1, 1024, 1024, 16, 128) == 1                # 16 key tiles: too short to cut
    assert fa.num_splits(1, 1024, 1024, 16, 128, causal=True) == 1
    assert fa.num_splits(1, 2048, 2048, 8, 128) == 1                 # hd128 small grids: 4-wave form
    assert fa.num_splits(1, 4096, 4096, 8, 128) == 1
    assert fa.num_splits(1, 2048, 2048, 8, 128, causal=True) == 2
    assert fa.num_splits(1, 4096, 4096, 8, 128, causal=True) == 3
    assert fa.num_splits(1, 4096, 4096, 16, 128, causal=True) == 1   # 256 workgroups
    assert fa.num_splits(1, 1024, 1024, 8, 512) == 1                 # no split-KV form at d = 512


@pytest.mark.parametrize("entry", ["fa_fwd_splitkv", "fa_fwd_splitkv_f16"])
def test_splitkv_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    assert _split(fn, q=0) == _lib.FA_ERR_NULL
    assert _split(fn, d=64) == _lib.FA_ERR_HEADDIM
    assert _split(fn, causal=1, Nk=17) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _split(fn, Hkv=3) == _lib.FA_ERR_SHAPE
    assert _split(fn, splits=0) == _lib.FA_ERR_SHAPE
    assert _split(fn, splits=257) == _lib.FA_ERR_SHAPE
    assert _split(fn, scale=math.nan) == _lib.FA_ERR_SCALE
    assert _split(fn, o=A + 2) == _lib.FA_ERR_ALIGN
    assert _split(fn, ws=0) == _lib.FA_ERR_WORKSPACE
    assert _split(fn, ws=A + 4) == _lib.FA_ERR_WORKSPACE
    assert _split(fn, wsb=4 * 2 * 8 * 300 * 129 * 4 - 1) == _lib.FA_ERR_WORKSPACE


def _fp8(**kw):
    a = dict(GOOD, **kw)
    return _lib.load().fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a.get("qs", 0.5),
                                  a.get("ks", 0.25), a.get("vs", 2.0), a["B"], a["Nq"], a["Nk"], a["Hq"],
                                  a["Hkv"], a["d"], a["causal"], ctypes.c_float(a["scale"]), None)


def test_fp8_rejects_before_any_hip_call():
    assert _fp8(k=0) == _lib.FA_ERR_NULL
    assert _fp8(d=64) == _lib.FA_ERR_HEADDIM
    assert _fp8(causal=1, Nk=17) == _lib.FA_ERR_CAUSAL_SHAPE
    assert _fp8(Hkv=3) == _lib.FA_ERR_SHAPE
    assert _fp8(scale=math.nan) == _lib.FA_ERR_SCALE
    for bad in (0.0, -1.0, math.inf, math.nan):
        assert _fp8(qs=bad) == _lib.FA_ERR_SCALE
        assert _fp8(ks=bad) == _lib.FA_ERR_SCALE
        assert _fp8(vs=bad) == _lib.FA_ERR_SCALE
    assert _fp8(v=A + 8) == _lib.FA_ERR_ALIGN
    assert _fp8(lse=A + 2) == _lib.FA_ERR_ALIGN
    assert _fp8(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 12, Nk=1 << 12) == _lib.FA_ERR_TOO_LARGE


def test_fp8_python_layer_checks_dtype():
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward_fp8(q, q, q)


def _var_ws_ok(a):
    return 4 * a["Hq"] * a["total_q"] * (a["d"] + 1) * 4


def _varlen_split(fn, **kw):
    a = dict(VGOOD, **kw)
    ws, wsb = a.get("ws", A + 0x900), a.get("wsb", _var_ws_ok(a))
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], ws, wsb, a["cu_q"], a["cu_k"], a["used"], a["B"],
              a["max_q"], a["total_q"], a["total_k"], a["Hq"], a["Hkv"], a["d"], a["causal"],
              ctypes.c_float(a["scale"]), a.get("splits", 4), None)


def _paged_split(fn, **kw):
    a = dict(VGOOD, **kw)
    ws, wsb = a.get("ws", A + 0x900), a.get("wsb", _var_ws_ok(a))
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], ws, wsb, a["cu_q"], a["used"], a["bt"], a["B"],
              a["max_q"], a["total_q"], a["num_pages"], a["page_size"], a["max_pages"], a["Hq"], a["Hkv"], a["d"],
              a["causal"], ctypes.c_float(a["scale"]), a.get("splits", 4), None)


def test_var_splitkv_workspace_size():
    lib = _lib.load()
    assert lib.fa_fwd_var_splitkv_workspace_bytes(300, 8, 128, 3) == 3 * 8 * 300 * 129 * 4
    assert lib.fa_fwd_var_splitkv_workspace_bytes(300, 8, 256, 1) == 8 * 300 * 257 * 4
    assert lib.fa_fwd_var_splitkv_workspace_bytes(300, 8, 512, 2) == 0
    assert lib.fa_fwd_var_splitkv_workspace_bytes(300, 8, 128, 0) == 0


@pytest.mark.parametrize("entry", ["fa_fwd_varlen_splitkv", "fa_fwd_varlen_splitkv_f16"])
def test_varlen_splitkv_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    for f in ("q", "cu_q", "cu_k"):
        assert _varlen_split(fn, **{f: 0}) == _lib.FA_ERR_NULL, f
    assert _varlen_split(fn, Hkv=3) == _lib.FA_ERR_SHAPE
    assert _varlen_split(fn, d=512) == _lib.FA_ERR_HEADDIM
    assert _varlen_split(fn, splits=0) == _lib.FA_ERR_SHAPE
    assert _varlen_split(fn, splits=257) == _lib.FA_ERR_SHAPE
    assert _varlen_split(fn, ws=0) == _lib.FA_ERR_WORKSPACE
    assert _varlen_split(fn, ws=A + 4) == _lib.FA_ERR_WORKSPACE
    a = dict(VGOOD)
    assert _varlen_split(fn, wsb=_var_ws_ok(a) - 1) == _lib.FA_ERR_WORKSPACE
    assert _varlen_split(fn, scale=math.nan) == _lib.FA_ERR_SCALE


@pytest.mark.parametrize("entry", ["fa_fwd_paged_splitkv", "fa_fwd_paged_splitkv_f16"])
def test_paged_splitkv_rejects_before_any_hip_call(entry):
    fn = getattr(_lib.load(), entry)
    for f in ("q", "used", "bt"):
        assert _paged_split(fn, **{f: 0}) == _lib.FA_ERR_NULL, f
    assert _paged_split(fn, page_size=100) == _lib.FA_ERR_PAGE
    assert _paged_split(fn, d=64) == _lib.FA_ERR_HEADDIM
    assert _paged_split(fn, splits=0) == _lib.FA_ERR_SHAPE
    assert _paged_split(fn, ws=0) == _lib.FA_ERR_WORKSPACE
    assert _paged_split(fn, o=A + 2) == _lib.FA_ERR_ALIGN


def test_var_num_splits_choice():
    assert fa.var_num_splits(128, 16, 32768, 8, 256) == 8        # decode over long caches
    assert fa.var_num_splits(128, 16, 32768, 8, 128) == 8
    assert fa.var_num_splits(8, 4096, 32768, 16, 128) == 0       # prefill: never
    assert fa.var_num_splits(8, 65, 32768, 16, 128) == 0
    assert fa.var_num_splits(4, 1, 512, 8, 256) == 0             # short caches: 16 tiles
    assert 2 <= fa.var_num_splits(4, 1, 2048, 8, 256) < 8        # 64 tiles
    assert fa.var_num_splits(4, 1, 2048, 8, 512) == 0            # unsupported head dim


def test_grid_order_setter_makes_no_hip_call():
    # a host-side setting only: returns FA_OK without a GPU, any values
    lib = _lib.load()
    for mul, add in ((7, 3), (0xFFFFFFFF, 0xFFFFFFFF), (0, 0)):
        assert lib.fa_set_grid_order(mul, add) == _lib.FA_OK
