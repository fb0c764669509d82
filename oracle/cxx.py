"""ctypes front of the C++ oracle (oracle/cpp/fp8ln_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may use it.  Every
step of the arithmetic runs in the C++ file; this module builds the library
with the host compiler (g++ -O2, OpenMP, no fast-math), marshals numpy arrays
and returns the results in the same shapes and dict keys as oracle.modules, so
the same pins run against both implementations.  The state containers
(Recipe, Meta) and the format names are oracle.modules' own: they carry no
arithmetic.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

from .codec import E4M3, E5M2
from .modules import (FORMAT_E4M3, FORMAT_E5M2, FORMAT_HYBRID, GELU_ERF, GELU_TANH, Recipe,
                      bwd_format, fwd_format, linear_bwd_meta, linear_fwd_meta, mlp_bwd_meta,
                      mlp_fwd_meta)
from .scaling import Meta

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "fp8ln_oracle.cpp")
LIB = os.path.join(HERE, "cpp", "liboracle.so")
CXX = os.environ.get("CXX_ORACLE", "g++")
FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]

_FMT = {E4M3: 0, E5M2: 1}

__all__ = ["build", "lib", "threads", "set_threads", "decode_table", "encode",
           "encode_f32_range", "encode_check_sign", "bf16_to_f64", "f64_to_bf16_bits",
           "scaling_update", "layernorm_fwd", "layernorm_bwd", "cast_amax", "fp8_gemm_tn",
           "gelu", "gelu_grad", "ln_cast_amax", "ln_linear_fwd", "ln_linear_bwd",
           "ln_mlp_fwd", "ln_mlp_bwd", "Recipe", "Meta", "fwd_format", "bwd_format",
           "linear_fwd_meta", "linear_bwd_meta", "mlp_fwd_meta", "mlp_bwd_meta",
           "FORMAT_E4M3", "FORMAT_HYBRID", "FORMAT_E5M2", "GELU_TANH", "GELU_ERF"]


def build(verbose: bool = False) -> str:
    """Compiles the C++ oracle into oracle/cpp/liboracle.so (host compiler only)."""
    tmp = LIB + ".tmp"
    cmd = [CXX, *FLAGS, "-o", tmp, SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


class _Meta(C.Structure):
    _fields_ = [("hist", C.c_void_p), ("scale", C.c_void_p), ("scale_inv", C.c_void_p),
                ("len", C.c_int32), ("n_slots", C.c_int32)]


_P = C.c_void_p
_I64 = C.c_int64
_I = C.c_int
_F = C.c_float
_D = C.c_double
_MP = C.POINTER(_Meta)

_SIGS = {
    "orc_decode_table": (None, [_I, _P]),
    "orc_encode": (None, [_P, _I64, _I, _P]),
    "orc_encode_f32_range": (None, [C.c_uint32, _I64, _I, _P]),
    "orc_encode_check_sign": (_I64, [_I, _I]),
    "orc_bf16_decode": (None, [_P, _I64, _P]),
    "orc_bf16_round": (None, [_P, _I64, _P]),
    "orc_scaling_update": (None, [_P, _P, _P, _I, _I, _P, _I]),
    "orc_record_amax": (None, [_P, _I, _F]),
    "orc_layernorm_fwd": (None, [_P, _I64, _I64, _P, _P, _D, _P, _P, _P]),
    "orc_layernorm_bwd": (None, [_P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P]),
    "orc_cast_amax": (_F, [_P, _I64, _F, _I, _P]),
    "orc_fp8_gemm_tn": (None, [_P, _I, _P, _I, _I64, _I64, _I64, _F, _F, _P, _P]),
    "orc_gelu": (None, [_P, _I64, _I, _P]),
    "orc_gelu_grad": (None, [_P, _I64, _I, _P]),
    "orc_ln_cast_amax": (_F, [_P, _I64, _I64, _P, _P, _D, _F, _I, _P, _P, _P]),
    "orc_ln_linear_fwd": (None, [_I, _D, _I64, _I64, _I64, _P, _P, _P, _P, _P, _MP, _I, _P, _P,
                                 _P, _P, _P, _P, _P, _P]),
    "orc_ln_linear_bwd": (None, [_I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _F, _P, _P, _MP,
                                 _MP, _P, _P, _P, _P, _P, _P, _P, _P]),
    "orc_ln_mlp_fwd": (None, [_I, _I, _D, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _MP,
                              _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "orc_ln_mlp_bwd": (None, [_I, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P, _P, _MP, _MP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P, _P]),
    "orc_num_threads": (_I, []),
    "orc_set_num_threads": (None, [_I]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded C++ oracle; built first if the library is missing or older
    than its source."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = C.CDLL(LIB)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def threads() -> int:
    return int(lib().orc_num_threads())


def set_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


# ---- primitives ------------------------------------------------------------------

def decode_table(fmt: str) -> np.ndarray:
    out = np.empty(256)
    lib().orc_decode_table(_FMT[fmt], _p(out))
    return out


def encode(values, fmt: str) -> np.ndarray:
    v = _arr(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_encode(_p(v), v.size, _FMT[fmt], _p(out))
    return out


def encode_f32_range(start: int, count: int, fmt: str, out=None) -> np.ndarray:
    if out is None:
        out = np.empty(count, dtype=np.uint8)
    lib().orc_encode_f32_range(start & 0xFFFFFFFF, count, _FMT[fmt], _p(out))
    return out


def encode_check_sign(fmt: str, negative: bool) -> int:
    """Violations of the exhaustive encoder check over every binary32 input of
    one sign (monotone, switching exactly at the midpoints, NaN -> 0x7F)."""
    return int(lib().orc_encode_check_sign(_FMT[fmt], int(negative)))


def bf16_to_f64(bits) -> np.ndarray:
    b = _arr(bits, np.uint16)
    out = np.empty(b.shape)
    lib().orc_bf16_decode(_p(b), b.size, _p(out))
    return out


def f64_to_bf16_bits(values) -> np.ndarray:
    v = _arr(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_round(_p(v), v.size, _p(out))
    return out


def _meta_fmts(meta: Meta) -> np.ndarray:
    return np.array([_FMT[f] for f in meta.formats], dtype=np.int32)


def _check_meta(meta: Meta):
    for a in (meta.history, meta.scale, meta.scale_inv):
        assert a.dtype == np.float32 and a.flags.c_contiguous


def _cmeta(meta: Meta) -> _Meta:
    _check_meta(meta)
    L, n = meta.history.shape
    return _Meta(meta.history.ctypes.data, meta.scale.ctypes.data, meta.scale_inv.ctypes.data,
                 L, n)


def scaling_update(meta: Meta, margin: int = 0) -> None:
    _check_meta(meta)
    L, n = meta.history.shape
    fm = _meta_fmts(meta)
    lib().orc_scaling_update(_p(meta.history), _p(meta.scale), _p(meta.scale_inv), L, n,
                             _p(fm), int(margin))


def layernorm_fwd(x, gamma, beta, eps: float):
    x = _arr(x, np.float64)
    rows, H = x.shape
    y = np.empty_like(x)
    mean, rstd = np.empty(rows), np.empty(rows)
    lib().orc_layernorm_fwd(_p(x), rows, H, _p(_arr(gamma, np.float64)),
                            _p(_arr(beta, np.float64)), float(eps), _p(y), _p(mean), _p(rstd))
    return y, mean, rstd


def layernorm_bwd(dy, x, gamma, mean, rstd):
    dy, x = _arr(dy, np.float64), _arr(x, np.float64)
    rows, H = x.shape
    dx = np.empty_like(x)
    dg, db = np.empty(H), np.empty(H)
    lib().orc_layernorm_bwd(_p(dy), _p(x), _p(_arr(gamma, np.float64)),
                            _p(_arr(mean, np.float64)), _p(_arr(rstd, np.float64)), rows, H,
                            _p(dx), _p(dg), _p(db))
    return dx, dg, db


def cast_amax(values, scale, fmt: str):
    v = _arr(values, np.float64)
    q = np.empty(v.shape, dtype=np.uint8)
    a = lib().orc_cast_amax(_p(v), v.size, float(np.float32(scale)), _FMT[fmt], _p(q))
    return q, np.float32(a)


def fp8_gemm_tn(a_codes, a_fmt, b_codes, b_fmt, sinv_a=1.0, sinv_b=1.0, bias=None):
    a, b = _arr(a_codes, np.uint8), _arr(b_codes, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    out = np.empty((M, N))
    bias = None if bias is None else _arr(bias, np.float64)
    lib().orc_fp8_gemm_tn(_p(a), _FMT[a_fmt], _p(b), _FMT[b_fmt], M, N, K,
                          float(np.float32(sinv_a)), float(np.float32(sinv_b)), _p(bias),
                          _p(out))
    return out


def gelu(h, activation=GELU_TANH):
    h = _arr(h, np.float64)
    out = np.empty_like(h)
    lib().orc_gelu(_p(h), h.size, int(activation), _p(out))
    return out


def gelu_grad(h, activation=GELU_TANH):
    h = _arr(h, np.float64)
    out = np.empty_like(h)
    lib().orc_gelu_grad(_p(h), h.size, int(activation), _p(out))
    return out


def ln_cast_amax(x_bits, gamma_bits, beta_bits, eps: float, scale, fmt: str, stats=True):
    """The standalone LayerNorm + cast + amax: (codes, amax, mean, rstd)."""
    x = _arr(x_bits, np.uint16)
    rows, H = x.shape
    q = np.empty((rows, H), dtype=np.uint8)
    mean = np.empty(rows) if stats else None
    rstd = np.empty(rows) if stats else None
    a = lib().orc_ln_cast_amax(_p(x), rows, H, _p(_arr(gamma_bits, np.uint16)),
                               _p(_arr(beta_bits, np.uint16)), float(eps),
                               float(np.float32(scale)), _FMT[fmt], _p(q), _p(mean), _p(rstd))
    return q, np.float32(a), mean, rstd


# ---- module steps (same arguments and results as oracle.modules) -----------------

def _opt_bits(b):
    return None if b is None else _arr(b, np.uint16)


def _amax_or_none(a):
    return None if np.isnan(a) else np.float32(a)


def ln_linear_fwd(recipe: Recipe, meta: Meta, x_bits, gamma_bits, beta_bits, w_bits,
                  bias_bits=None, cached_w=None):
    x, w = _arr(x_bits, np.uint16), _arr(w_bits, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N))
    ln_q = np.empty((M, K), dtype=np.uint8)
    y = np.empty((M, K))
    mean, rstd = np.empty(M), np.empty(M)
    amaxes = np.zeros(2, dtype=np.float32)
    w_sinv = np.zeros(1, dtype=np.float32)
    if cached_w is not None:
        w_q = _arr(cached_w[0], np.uint8).copy()
        w_sinv[0] = np.float32(cached_w[1])
    else:
        w_q = np.empty((N, K), dtype=np.uint8)
    bias = _opt_bits(bias_bits)
    cm = _cmeta(meta)
    lib().orc_ln_linear_fwd(recipe.format, recipe.eps64, M, K, N, _p(x),
                            _p(_arr(gamma_bits, np.uint16)), _p(_arr(beta_bits, np.uint16)),
                            _p(w), _p(bias), C.byref(cm), int(cached_w is not None), _p(out),
                            _p(ln_q), _p(w_q), _p(w_sinv), _p(y), _p(mean), _p(rstd),
                            _p(amaxes))
    ctx = dict(ln_q=ln_q, w_q=w_q, w_sinv=np.float32(w_sinv[0]), mean=mean, rstd=rstd, y=y,
               ln_amax=np.float32(amaxes[0]),
               w_amax=None if cached_w is not None else np.float32(amaxes[1]))
    return out, ctx


def ln_linear_bwd(recipe: Recipe, meta_fwd: Meta, meta_bwd: Meta, dy_bits, ctx, x_bits,
                  gamma_bits):
    dy, x = _arr(dy_bits, np.uint16), _arr(x_bits, np.uint16)
    M, N = dy.shape
    K = x.shape[1]
    dx, dln = np.empty((M, K)), np.empty((M, K))
    dg, db = np.empty(K), np.empty(K)
    dw, dbias = np.empty((N, K)), np.empty(N)
    dy_q = np.empty((M, N), dtype=np.uint8)
    dy_amax = np.zeros(1, dtype=np.float32)
    cf, cb = _cmeta(meta_fwd), _cmeta(meta_bwd)
    lib().orc_ln_linear_bwd(recipe.format, M, K, N, _p(dy), _p(x),
                            _p(_arr(gamma_bits, np.uint16)), _p(_arr(ctx["ln_q"], np.uint8)),
                            _p(_arr(ctx["w_q"], np.uint8)), float(ctx["w_sinv"]),
                            _p(_arr(ctx["mean"], np.float64)), _p(_arr(ctx["rstd"], np.float64)),
                            C.byref(cf), C.byref(cb), _p(dx), _p(dg), _p(db), _p(dw), _p(dbias),
                            _p(dln), _p(dy_q), _p(dy_amax))
    return dict(dx=dx, dgamma=dg, dbeta=db, dw=dw, dbias=dbias, dy_q=dy_q,
                dy_amax=np.float32(dy_amax[0]), dln=dln)


def ln_mlp_fwd(recipe: Recipe, meta: Meta, x_bits, gamma_bits, beta_bits, w1_bits, b1_bits,
               w2_bits, b2_bits, cached_w=None):
    x, w1, w2 = _arr(x_bits, np.uint16), _arr(w1_bits, np.uint16), _arr(w2_bits, np.uint16)
    M, H = x.shape
    F = w1.shape[0]
    out = np.empty((M, H))
    ln_q = np.empty((M, H), dtype=np.uint8)
    h, g = np.empty((M, F)), np.empty((M, F))
    h_bits = np.empty((M, F), dtype=np.uint16)
    g_q = np.empty((M, F), dtype=np.uint8)
    y = np.empty((M, H))
    mean, rstd = np.empty(M), np.empty(M)
    amaxes = np.zeros(4, dtype=np.float32)
    w_sinv = np.zeros(2, dtype=np.float32)
    if cached_w is not None:
        (c1, s1), (c2, s2) = cached_w
        w1_q, w2_q = _arr(c1, np.uint8).copy(), _arr(c2, np.uint8).copy()
        w_sinv[:] = [np.float32(s1), np.float32(s2)]
    else:
        w1_q = np.empty((F, H), dtype=np.uint8)
        w2_q = np.empty((H, F), dtype=np.uint8)
    cm = _cmeta(meta)
    lib().orc_ln_mlp_fwd(recipe.format, recipe.activation, recipe.eps64, M, H, F, _p(x),
                         _p(_arr(gamma_bits, np.uint16)), _p(_arr(beta_bits, np.uint16)),
                         _p(w1), _p(_opt_bits(b1_bits)), _p(w2), _p(_opt_bits(b2_bits)),
                         C.byref(cm), int(cached_w is not None), _p(out), _p(ln_q), _p(w1_q),
                         _p(w2_q), _p(w_sinv), _p(h), _p(h_bits), _p(g), _p(g_q), _p(y),
                         _p(mean), _p(rstd), _p(amaxes))
    reuse = cached_w is not None
    ctx = dict(ln_q=ln_q, w1_q=w1_q, w2_q=w2_q, w1_sinv=np.float32(w_sinv[0]),
               w2_sinv=np.float32(w_sinv[1]), h=h, h_bits=h_bits, g=g, g_q=g_q, mean=mean,
               rstd=rstd, y=y, ln_amax=np.float32(amaxes[0]),
               w1_amax=None if reuse else np.float32(amaxes[1]),
               w2_amax=None if reuse else np.float32(amaxes[3]), g_amax=np.float32(amaxes[2]))
    return out, ctx


def ln_mlp_bwd(recipe: Recipe, meta_fwd: Meta, meta_bwd: Meta, dy_bits, ctx, x_bits,
               gamma_bits):
    dy, x = _arr(dy_bits, np.uint16), _arr(x_bits, np.uint16)
    M, H = dy.shape
    F = ctx["h_bits"].shape[1]
    dx, dln = np.empty((M, H)), np.empty((M, H))
    dgam, dbet = np.empty(H), np.empty(H)
    dw1, db1 = np.empty((F, H)), np.empty(F)
    dw2, db2 = np.empty((H, F)), np.empty(H)
    dg, dh = np.empty((M, F)), np.empty((M, F))
    dy_q = np.empty((M, H), dtype=np.uint8)
    dh_q = np.empty((M, F), dtype=np.uint8)
    amaxes = np.zeros(2, dtype=np.float32)
    w_sinv = np.array([ctx["w1_sinv"], ctx["w2_sinv"]], dtype=np.float32)
    cf, cb = _cmeta(meta_fwd), _cmeta(meta_bwd)
    lib().orc_ln_mlp_bwd(recipe.format, recipe.activation, M, H, F, _p(dy), _p(x),
                         _p(_arr(gamma_bits, np.uint16)), _p(_arr(ctx["ln_q"], np.uint8)),
                         _p(_arr(ctx["w1_q"], np.uint8)), _p(_arr(ctx["w2_q"], np.uint8)),
                         _p(w_sinv), _p(_arr(ctx["h_bits"], np.uint16)),
                         _p(_arr(ctx["g_q"], np.uint8)), _p(_arr(ctx["mean"], np.float64)),
                         _p(_arr(ctx["rstd"], np.float64)), C.byref(cf), C.byref(cb), _p(dx),
                         _p(dgam), _p(dbet), _p(dw1), _p(db1), _p(dw2), _p(db2), _p(dg), _p(dh),
                         _p(dy_q), _p(dh_q), _p(dln), _p(amaxes))
    return dict(dx=dx, dgamma=dgam, dbeta=dbet, dw1=dw1, db1=db1, dw2=dw2, db2=db2, dy_q=dy_q,
                dy_amax=np.float32(amaxes[0]), dh=dh, dh_q=dh_q, dh_amax=np.float32(amaxes[1]),
                dg=dg, dln=dln)
