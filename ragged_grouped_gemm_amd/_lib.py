"""ctypes loader of ``libmoe_mi355x.so`` and the C structures of ``include/moe.h``.

The library is built in-tree by ``python -m ragged_grouped_gemm_amd.build``.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_E4M3, MOE_E2M1 = 0, 1, 2, 3
ACT = {"swiglu": 0, "geglu": 1, "srelu": 2}
SCORE = {"softmax": 0, "sigmoid": 1}
MOE_BWD_DGRAD, MOE_BWD_WGRAD = 0, 1
ERRBIT_NAN_LOGIT, ERRBIT_BAD_EXPERT = 1, 2

c_int, c_float, c_void_p, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MxT(ctypes.Structure):
    """moe_mx_t: E4M3 codes [rows, ld], E8M0 scales [rows, ld / 32]."""
    _fields_ = [("data", c_void_p), ("scale", c_void_p), ("ld", ctypes.c_int64)]


_PMX = ctypes.POINTER(MxT)


class GluFwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("dtype", c_int), ("xp", c_void_p), ("w1p", c_void_p),
                ("b1p", c_void_p), ("offsets", c_void_p), ("E", c_int), ("R", c_int),
                ("d", c_int), ("f", c_int), ("act", c_int), ("clamp", c_float),
                ("alpha", c_float), ("gelu_tanh", c_int), ("h_out", c_void_p),
                ("a_out", c_void_p), ("max_cus", c_int), ("xp_mx", _PMX), ("w1_mx", _PMX),
                ("a_row", _PMX), ("a_col", _PMX), ("pad_offsets", c_void_p),
                ("src_row", c_void_p), ("src_rows", c_int), ("row_scale", c_void_p)]


class GemmFwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("dtype", c_int), ("a", c_void_p), ("w", c_void_p),
                ("b", c_void_p), ("offsets", c_void_p), ("E", c_int), ("R", c_int),
                ("N", c_int), ("K", c_int), ("y", c_void_p), ("max_cus", c_int),
                ("a_mx", _PMX), ("w_mx", _PMX), ("y_mx", _PMX)]


class GluBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("dtype", c_int), ("dy", c_void_p), ("w2", c_void_p),
                ("h", c_void_p), ("offsets", c_void_p), ("E", c_int), ("R", c_int),
                ("d", c_int), ("f", c_int), ("act", c_int), ("clamp", c_float),
                ("alpha", c_float), ("gelu_tanh", c_int), ("dh", c_void_p),
                ("max_cus", c_int), ("dy_mx", _PMX), ("w2t_mx", _PMX), ("dh_row", _PMX),
                ("dh_col", _PMX), ("pad_offsets", c_void_p), ("w2t", c_void_p),
                ("row_scale", c_void_p), ("d_row_scale", c_void_p), ("ws", c_void_p),
                ("ws_bytes", c_size_t)]


class GemmBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", c_size_t), ("dtype", c_int), ("mode", c_int), ("g", c_void_p),
                ("a", c_void_p), ("w", c_void_p), ("offsets", c_void_p), ("E", c_int),
                ("R", c_int), ("N", c_int), ("K", c_int), ("out", c_void_p), ("db", c_void_p),
                ("accumulate", c_int), ("max_cus", c_int), ("g_mx", _PMX), ("a_mx", _PMX),
                ("w_mx", _PMX), ("pad_offsets", c_void_p), ("a_src_row", c_void_p),
                ("a_src_rows", c_int), ("out_mx", _PMX), ("wt", c_void_p)]


_SIGS = {
    "moe_version": (ctypes.c_char_p, []),
    "moe_status_string": (ctypes.c_char_p, [c_int]),
    "moe_glu_granularity": (c_int, []),
    "moe_route_topk": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                               c_void_p, c_void_p]),
    "moe_route_topk_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                   c_int, c_void_p, c_void_p]),
    "moe_router_topk": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "moe_router_bwd": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int,
                               c_void_p, c_int, c_void_p, c_void_p]),
    "moe_permute_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "moe_permute": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_int, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                            c_void_p, c_void_p]),
    "moe_permute_noalloc": (c_int, [c_void_p, c_int, c_int, c_int, c_void_p, c_int, c_int,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
    "moe_permute_rows": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "moe_glu_bwd_workspace_size": (c_size_t, [c_int, c_int]),
    "moe_repack_glu_weights": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                       c_void_p, c_void_p, c_void_p]),
    "moe_transpose_weights": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_grouped_gemm_glu_fwd": (c_int, [ctypes.POINTER(GluFwdArgs), c_void_p]),
    "moe_grouped_gemm_fwd": (c_int, [ctypes.POINTER(GemmFwdArgs), c_void_p]),
    "moe_grouped_gemm_glu_bwd": (c_int, [ctypes.POINTER(GluBwdArgs), c_void_p]),
    "moe_grouped_gemm_bwd": (c_int, [ctypes.POINTER(GemmBwdArgs), c_void_p]),
    "moe_unpermute_combine": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                      c_void_p, c_void_p]),
    "moe_unpermute_combine_bwd": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int,
                                          c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "moe_mx_col_len": (ctypes.c_int64, [c_int, c_int]),
    "moe_mx_col_ld": (ctypes.c_int64, [c_int, c_int, c_int]),
    "moe_mx_quantize": (c_int, [c_void_p, c_int, ctypes.c_int64, c_int, _PMX, c_void_p]),
    "moe_mx_quantize_transpose": (c_int, [c_void_p, c_int, c_int, c_int, c_int, _PMX, c_void_p]),
    "moe_mx_quantize_experts": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                        c_void_p, c_void_p, c_int, c_int, c_int, _PMX, _PMX,
                                        c_void_p]),
    "moe_unpermute_combine_mx": (c_int, [_PMX, c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                         c_void_p, c_int, c_void_p]),
    "moe_mxfp4_quantize": (c_int, [c_void_p, c_int, ctypes.c_int64, c_int, _PMX, c_void_p]),
    "moe_mxfp4_quantize_transpose": (c_int, [c_void_p, c_int, c_int, c_int, c_int, _PMX,
                                             c_void_p]),
    "moe_mxfp4_quantize_experts": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int,
                                           c_void_p, c_void_p, c_int, c_int, c_int, _PMX, _PMX,
                                           c_void_p]),
}

_lib = None


def header_functions(path: str = HEADER):
    """Names of the functions declared in the C header."""
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m ragged_grouped_gemm_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoEError(RuntimeError):
    pass


def check(status: int, what: str):
    if status != MOE_OK:
        name = load().moe_status_string(status).decode()
        raise MoEError(f"{what} failed: {name} ({status})")
