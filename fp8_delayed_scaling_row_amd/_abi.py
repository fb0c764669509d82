"""ctypes view of include/fp8ln.h and the loader of libfp8ln.so.

The library must be built (python -m fp8_delayed_scaling_row_amd.build); there is
no fallback: loading fails loudly when the shared object is missing.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8ln.so")

FP8LN_OK = 0
FP8LN_ERR_INVALID_ARG = -1
FP8LN_ERR_UNSUPPORTED = -2
FP8LN_ERR_HIP = -3

FORMAT_E4M3 = 0
FORMAT_HYBRID = 1
FORMAT_E5M2 = 2

E4M3 = 0
E5M2 = 1

DTYPE_BF16 = 0
DTYPE_F32 = 1

GELU_TANH = 0
GELU_ERF = 1

META_FORWARD = 0
META_BACKWARD = 1

STEP_WS_BYTES = 64   # FP8LN_STEP_WS_BYTES

OP_CAST_AMAX = 0
OP_LAYERNORM_BWD = 1
OP_LN_LINEAR_BWD = 2
OP_LN_MLP_BWD = 3
OP_GEMM_DGELU_FP8 = 4
OP_LINEAR_BWD = 5
OP_LN_LINEAR_BWD_BF16 = 6
OP_TRANSPOSE_BF16 = 7
OP_LN_MLP_BWD_BF16 = 8


class Recipe(C.Structure):
    _fields_ = [("format", C.c_int32), ("amax_history_len", C.c_int32),
                ("margin", C.c_int32), ("ln_eps", C.c_float), ("activation", C.c_int32)]


class MetaStruct(C.Structure):
    _fields_ = [("amax_history", C.c_void_p), ("scale", C.c_void_p),
                ("scale_inv", C.c_void_p), ("n_slots", C.c_int32), ("kind", C.c_int32)]


class LinearCtxStruct(C.Structure):
    _fields_ = [("ln_q", C.c_void_p), ("ln_qt", C.c_void_p), ("w_q", C.c_void_p),
                ("w_qt", C.c_void_p), ("mean", C.c_void_p), ("rstd", C.c_void_p),
                ("w_scale_inv", C.c_void_p), ("reuse_weight_codes", C.c_int32)]


class MlpCtxStruct(C.Structure):
    _fields_ = [("ln_q", C.c_void_p), ("ln_qt", C.c_void_p), ("w1_q", C.c_void_p),
                ("w1_qt", C.c_void_p), ("w2_q", C.c_void_p), ("w2_qt", C.c_void_p),
                ("h", C.c_void_p), ("g_q", C.c_void_p), ("g_qt", C.c_void_p),
                ("mean", C.c_void_p), ("rstd", C.c_void_p), ("w_scale_inv", C.c_void_p),
                ("reuse_weight_codes", C.c_int32)]


_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_SZ = C.c_size_t
_RP = C.POINTER(Recipe)
_MP = C.POINTER(MetaStruct)

# name -> (restype, argtypes); the order of include/fp8ln.h
SIGNATURES = {
    "fp8ln_status_string": (C.c_char_p, [C.c_int]),
    "fp8ln_last_error": (C.c_char_p, []),
    "fp8ln_check_support": (C.c_int, [C.c_int, C.c_char_p, _SZ]),
    "fp8ln_workspace_size": (_SZ, [_I32, _I64, _I64, _I64]),
    "fp8ln_meta_init": (C.c_int, [_RP, _MP, _P]),
    "fp8ln_scaling_update": (C.c_int, [_RP, _MP, _P]),
    "fp8ln_scaling_update_batch": (C.c_int, [_RP, C.POINTER(MetaStruct), _I32, _P]),
    "fp8ln_ln_cast_amax": (C.c_int, [_RP, _I64, _I64, _I32, _P, _P, _P, _I32, _P, _P, _P, _P,
                                     _P, _P, _P]),
    "fp8ln_cast_amax": (C.c_int, [_I64, _I64, _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp8ln_encode_range": (C.c_int, [C.c_uint32, _I64, _I32, _P, _P]),
    "fp8ln_stream_probe": (C.c_int, [_I64, _P, _P, _P]),
    "fp8ln_gemm": (C.c_int, [_I64, _I64, _I64, _P, _I32, _P, _I32, _P, _P, _P, _I32, _P, _P]),
    "fp8ln_gemm_gelu_fp8": (C.c_int, [_I64, _I64, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P, _P,
                                      _P, _I32, _P, _P, _I32, _P]),
    "fp8ln_gemm_dgelu": (C.c_int, [_I64, _I64, _I64, _P, _I32, _P, _I32, _P, _P, _P, _P, _I32,
                                   _P]),
    "fp8ln_gemm_dgelu_fp8": (C.c_int, [_I64, _I64, _I64, _P, _I32, _P, _I32, _P, _P, _P, _I32, _P,
                                       _P, _P, _P, _P, _I32, _P, _SZ, _P]),
    "fp8ln_layernorm_bwd": (C.c_int, [_I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fp8ln_gemm_bf16": (C.c_int, [_I64, _I64, _I64, _P, _P, _P, _I32, _P, _P]),
    "fp8ln_gemm_gelu_bf16": (C.c_int, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _I32, _P]),
    "fp8ln_gemm_dgelu_bf16": (C.c_int, [_I64, _I64, _I64, _P, _P, _P, _P, _I32, _P]),
    "fp8ln_ln_mlp_bwd_bf16": (C.c_int, [_I64, _I64, _I64, _I32] + [_P] * 18 + [_SZ, _P]),
    "fp8ln_transpose_bf16": (C.c_int, [_I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "fp8ln_ln_linear_fwd_bf16": (C.c_int, [_I64, _I64, _I64, C.c_float, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P]),
    "fp8ln_ln_linear_bwd_bf16": (C.c_int, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _SZ, _P]),
    "fp8ln_ln_mlp_fwd_bf16": (C.c_int, [_I64, _I64, _I64, C.c_float, _I32, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "fp8ln_layernorm_fwd": (C.c_int, [_I64, _I64, C.c_float, _P, _P, _P, _P, _P, _P, _P]),
    "fp8ln_layernorm_bwd_bf16": (C.c_int, [_I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                           _P]),
    "fp8ln_linear_fwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _MP,
                                   C.POINTER(LinearCtxStruct), _P]),
    "fp8ln_linear_bwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, C.POINTER(LinearCtxStruct),
                                   _MP, _MP, _P, _P, _P, _P, _SZ, _P]),
    "fp8ln_ln_linear_fwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _MP,
                                      C.POINTER(LinearCtxStruct), _P]),
    "fp8ln_ln_linear_fwd_step": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P,
                                           _MP, C.POINTER(LinearCtxStruct), _P, _P]),
    "fp8ln_ln_linear_bwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P,
                                      C.POINTER(LinearCtxStruct), _MP, _MP, _P, _P, _P, _P, _P,
                                      _P, _SZ, _P]),
    "fp8ln_ln_linear_bwd_step": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P,
                                           C.POINTER(LinearCtxStruct), _MP, _MP, _P, _P, _P, _P,
                                           _P, _P, _SZ, _P, _P]),
    "fp8ln_ln_linear_bwd_noalloc": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P,
                                              C.POINTER(LinearCtxStruct), _MP, _MP, _P, _P, _P,
                                              _P, _P, _P]),
    "fp8ln_ln_mlp_fwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _MP, C.POINTER(MlpCtxStruct), _P]),
    "fp8ln_ln_mlp_fwd_step": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _MP, C.POINTER(MlpCtxStruct), _P, _P]),
    "fp8ln_ln_mlp_bwd": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P,
                                   C.POINTER(MlpCtxStruct), _MP, _MP, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _SZ, _P]),
    "fp8ln_ln_mlp_bwd_step": (C.c_int, [_RP, _I64, _I64, _I64, _I32, _P, _P, _P,
                                        C.POINTER(MlpCtxStruct), _MP, _MP, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _SZ, _P, _P]),
}

_lib = None


class Fp8lnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> C.CDLL:
    """The loaded libfp8ln.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m fp8_delayed_scaling_row_amd.build` (there is no fallback path)")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != FP8LN_OK:
        L = lib()
        msg = L.fp8ln_last_error().decode() or L.fp8ln_status_string(status).decode()
        raise Fp8lnError(status, msg)
