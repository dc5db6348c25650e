"""ctypes loader for libfa.so (the HIP library behind include/fa_fwd.h).

Argument marshalling only: every step of the forward pass runs in the library's kernels.
There is no fallback: if the library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "fa_fwd.h")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEADDIM = -3
FA_ERR_CAUSAL_SHAPE = -4
FA_ERR_SCALE = -5
FA_ERR_ALIGN = -6
FA_ERR_TOO_LARGE = -7
FA_ERR_LAUNCH = -8
FA_ERR_WORKSPACE = -9
FA_ERR_PAGE = -10
FA_ERR_SCRATCH = -11
FA_BWD_NOALLOC_MAX_ROWS = 8 << 20  # include/fa_fwd.h

_lib = None

_I = ctypes.c_int
_P = ctypes.c_void_p
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
_CHECK_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float]
# q, k, v, o, lse, cu_q, cu_k, seqused, B, max_seqlen_q, total_q, total_k, Hq, Hkv, d, causal, scale, stream
_VARLEN_ARGS = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
# q, kc, vc, o, lse, cu_q, seqused, block_table, B, max_seqlen_q, total_q, num_pages, page_size,
# max_pages, Hq, Hkv, d, causal, scale, stream
_PAGED_ARGS = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
# q, k, v, o, lse, workspace, workspace_bytes, B, Nq, Nk, Hq, Hkv, d, causal, scale, num_splits, stream
_SPLIT_ARGS = [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P]
_BWD_ARGS = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I, _I, _I, _I, _I, _I, _I,
             ctypes.c_float, _P]
# q, k, v, o, lse, workspace, workspace_bytes, cu_q, cu_k, seqused, B, max_seqlen_q, total_q,
# total_k, Hq, Hkv, d, causal, scale, num_splits, stream
_VARLEN_SPLIT_ARGS = [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                      ctypes.c_float, _I, _P]
# q, kc, vc, o, lse, workspace, workspace_bytes, cu_q, seqused, block_table, B, max_seqlen_q,
# total_q, num_pages, page_size, max_pages, Hq, Hkv, d, causal, scale, num_splits, stream
_PAGED_SPLIT_ARGS = [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                     _I, ctypes.c_float, _I, _P]


def load():
    """Load libfa.so once; raise if it has not been built. FA_LIB may name another build of
    the same sources (the host-only AddressSanitizer build runs the contract tests)."""
    global _lib
    if _lib is None:
        path = os.environ.get("FA_LIB") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m exact_attention_06_amd.build`")
        lib = ctypes.CDLL(path)
        for name in ("fa_fwd", "fa_fwd_f16"):
            fn = getattr(lib, name)
            fn.argtypes = _FWD_ARGS
            fn.restype = _I
        for names, args in ((("fa_fwd_varlen", "fa_fwd_varlen_f16"), _VARLEN_ARGS),
                            (("fa_fwd_paged", "fa_fwd_paged_f16"), _PAGED_ARGS)):
            for name in names:
                fn = getattr(lib, name)
                fn.argtypes = args
                fn.restype = _I
        lib.fa_fwd_fp8.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                   _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
        lib.fa_fwd_fp8.restype = _I
        for name in ("fa_fwd_splitkv", "fa_fwd_splitkv_f16"):
            fn = getattr(lib, name)
            fn.argtypes = _SPLIT_ARGS
            fn.restype = _I
        for name in ("fa_fwd_varlen_splitkv", "fa_fwd_varlen_splitkv_f16"):
            fn = getattr(lib, name)
            fn.argtypes = _VARLEN_SPLIT_ARGS
            fn.restype = _I
        for name in ("fa_fwd_paged_splitkv", "fa_fwd_paged_splitkv_f16"):
            fn = getattr(lib, name)
            fn.argtypes = _PAGED_SPLIT_ARGS
            fn.restype = _I
        lib.fa_fwd_var_num_splits.argtypes = [_I, _I, _I, _I, _I]
        lib.fa_fwd_var_num_splits.restype = _I
        lib.fa_fwd_var_splitkv_workspace_bytes.argtypes = [_I, _I, _I, _I]
        lib.fa_fwd_var_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_splitkv_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_num_splits.argtypes = [_I, _I, _I, _I, _I, _I]
        lib.fa_fwd_num_splits.restype = _I
        for name in ("fa_bwd", "fa_bwd_f16"):
            fn = getattr(lib, name)
            fn.argtypes = _BWD_ARGS
            fn.restype = _I
        # q, k, v, o, lse, dout, dq, dk, dv, B, Nq, Nk, Hq, Hkv, d, causal, scale, stream
        lib.fa_bwd_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                       ctypes.c_float, _P]
        lib.fa_bwd_noalloc.restype = _I
        lib.fa_bwd_workspace_bytes.argtypes = [_I, _I, _I]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_check.argtypes = _CHECK_ARGS
        lib.fa_fwd_check.restype = _I
        lib.fa_strerror.argtypes = [_I]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_set_grid_order.argtypes = [ctypes.c_uint, ctypes.c_uint]
        lib.fa_set_grid_order.restype = _I
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load().fa_strerror(int(code)).decode()


def header_symbols():
    """Function names declared in include/fa_fwd.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(fa_\w+)\s*\(", text, flags=re.M)))
