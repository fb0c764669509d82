"""Python binding of libfp8ln: the C-ABI calls with torch tensors as buffers.

Every function marshals tensor pointers and sizes and calls the entry point of
the same name in include/fp8ln.h on torch's current HIP stream.  No step of the
computation happens here; torch only provides device memory and the stream.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _abi
from ._abi import (DTYPE_BF16, DTYPE_F32, E4M3, E5M2, FORMAT_E4M3, FORMAT_E5M2, FORMAT_HYBRID,
                   GELU_ERF, GELU_TANH,
                   META_BACKWARD, META_FORWARD, OP_CAST_AMAX, OP_LAYERNORM_BWD, OP_LN_LINEAR_BWD,
                   OP_LN_MLP_BWD, OP_GEMM_DGELU_FP8, OP_LINEAR_BWD, Fp8lnError, check, lib)

__all__ = [
    "Recipe", "Meta", "LinearCtx", "MlpCtx", "Fp8lnError", "FORMAT_E4M3", "FORMAT_HYBRID",
    "FORMAT_E5M2", "GELU_TANH", "GELU_ERF", "E4M3", "E5M2", "META_FORWARD", "META_BACKWARD", "OP_CAST_AMAX",
    "OP_LAYERNORM_BWD", "OP_LN_LINEAR_BWD", "OP_LN_MLP_BWD", "OP_GEMM_DGELU_FP8", "OP_LINEAR_BWD",
    "check_support", "workspace_size", "meta_init",
    "scaling_update", "ln_cast_amax", "cast_amax", "encode_range", "stream_probe", "gemm", "gemm_gelu_fp8",
    "gemm_dgelu", "gemm_dgelu_fp8", "layernorm_bwd", "layernorm_fwd", "layernorm_bwd_bf16",
    "linear_fwd", "linear_bwd", "gemm_bf16", "gemm_gelu_bf16", "transpose_bf16",
    "ln_linear_fwd_bf16", "ln_linear_bwd_bf16", "ln_mlp_fwd_bf16", "ln_mlp_bwd_bf16",
    "gemm_dgelu_bf16",
    "ln_linear_fwd", "ln_linear_bwd", "ln_linear_bwd_noalloc", "ln_mlp_fwd", "ln_mlp_bwd", "fwd_fp8", "bwd_fp8",
]


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _opt(t, dtype, shape, name):
    if t is not None:
        _need(t, dtype, shape, name)


@dataclass
class Recipe:
    """DelayedScaling recipe: format, amax_history_len, margin, LayerNorm eps, and
    the LayerNormMLP activation (GELU_TANH or GELU_ERF)."""
    format: int = FORMAT_HYBRID
    amax_history_len: int = 16
    margin: int = 0
    ln_eps: float = 1e-5
    activation: int = 0

    def as_c(self) -> _abi.Recipe:
        return _abi.Recipe(self.format, self.amax_history_len, self.margin, self.ln_eps,
                           self.activation)


def fwd_fp8(recipe: Recipe) -> int:
    return E5M2 if recipe.format == FORMAT_E5M2 else E4M3


def bwd_fp8(recipe: Recipe) -> int:
    return E4M3 if recipe.format == FORMAT_E4M3 else E5M2


class Meta:
    """One direction's FP8 state of one module: history [L][n_slots], scale and
    scale_inv [n_slots], all float32 device tensors."""

    def __init__(self, recipe: Recipe, n_slots: int, kind: int, device="cuda", init=True):
        self.recipe = recipe
        self.kind = kind
        self.history = torch.zeros((recipe.amax_history_len, n_slots), dtype=torch.float32,
                                   device=device)
        self.scale = torch.ones(n_slots, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(n_slots, dtype=torch.float32, device=device)
        if init:
            meta_init(recipe, self)

    @property
    def n_slots(self) -> int:
        return self.history.shape[1]

    def as_c(self) -> _abi.MetaStruct:
        return _abi.MetaStruct(self.history.data_ptr(), self.scale.data_ptr(),
                               self.scale_inv.data_ptr(), self.n_slots, self.kind)

    def amax_ptr(self, slot: int) -> int:
        """Address of history row 0 for `slot` (where the step records its amax)."""
        return self.history.data_ptr() + 4 * slot

    def state_dict(self) -> dict:
        """Host copy of the state (the per-tensor scale, its inverse and the amax
        history, as fp8_meta keeps them), for a checkpoint."""
        return dict(amax_history=self.history.cpu().clone(), scale=self.scale.cpu().clone(),
                    scale_inv=self.scale_inv.cpu().clone())

    def load_state_dict(self, d: dict) -> None:
        """Restore a state_dict() (same history length and slot count)."""
        if tuple(d["amax_history"].shape) != tuple(self.history.shape):
            raise ValueError("history shape differs from this state block's")
        self.history.copy_(d["amax_history"])
        self.scale.copy_(d["scale"])
        self.scale_inv.copy_(d["scale_inv"])


class LinearCtx:
    """What LayerNormLinear's (or Linear's) forward saves for its backward; for
    Linear, ln_q / ln_qt hold the input's codes and mean / rstd go unused."""

    def __init__(self, tokens: int, in_features: int, out_features: int, training=True,
                 device="cuda"):
        u8 = dict(dtype=torch.uint8, device=device)
        self.ln_q = torch.empty((tokens, in_features), **u8)
        self.w_q = torch.empty((out_features, in_features), **u8)
        self.ln_qt = torch.empty((in_features, tokens), **u8) if training else None
        self.w_qt = torch.empty((in_features, out_features), **u8) if training else None
        self.mean = torch.empty(tokens, dtype=torch.float32, device=device)
        self.rstd = torch.empty(tokens, dtype=torch.float32, device=device)
        # scale_inv of the cached weight codes; set reuse_weight_codes to skip the
        # weight cast while the weight is unchanged (FP8 weight storage)
        self.w_scale_inv = torch.ones(1, dtype=torch.float32, device=device)
        self.reuse_weight_codes = False

    def as_c(self) -> _abi.LinearCtxStruct:
        p = lambda t: None if t is None else t.data_ptr()
        return _abi.LinearCtxStruct(p(self.ln_q), p(self.ln_qt), p(self.w_q), p(self.w_qt),
                                    p(self.mean), p(self.rstd), p(self.w_scale_inv),
                                    int(bool(self.reuse_weight_codes)))


class MlpCtx:
    """What LayerNormMLP's forward saves for its backward."""

    def __init__(self, tokens: int, hidden: int, ffn: int, training=True, device="cuda"):
        u8 = dict(dtype=torch.uint8, device=device)
        self.ln_q = torch.empty((tokens, hidden), **u8)
        self.w1_q = torch.empty((ffn, hidden), **u8)
        self.w2_q = torch.empty((hidden, ffn), **u8)
        self.g_q = torch.empty((tokens, ffn), **u8)
        self.ln_qt = torch.empty((hidden, tokens), **u8) if training else None
        self.w1_qt = torch.empty((hidden, ffn), **u8) if training else None
        self.w2_qt = torch.empty((ffn, hidden), **u8) if training else None
        self.g_qt = torch.empty((ffn, tokens), **u8) if training else None
        self.h = torch.empty((tokens, ffn), dtype=torch.bfloat16, device=device) if training else None
        self.mean = torch.empty(tokens, dtype=torch.float32, device=device)
        self.rstd = torch.empty(tokens, dtype=torch.float32, device=device)
        self.w_scale_inv = torch.ones(2, dtype=torch.float32, device=device)   # fc1, fc2
        self.reuse_weight_codes = False

    def as_c(self) -> _abi.MlpCtxStruct:
        p = lambda t: None if t is None else t.data_ptr()
        return _abi.MlpCtxStruct(p(self.ln_q), p(self.ln_qt), p(self.w1_q), p(self.w1_qt),
                                 p(self.w2_q), p(self.w2_qt), p(self.h), p(self.g_q),
                                 p(self.g_qt), p(self.mean), p(self.rstd), p(self.w_scale_inv),
                                 int(bool(self.reuse_weight_codes)))


# ---- library -----------------------------------------------------------------

def check_support(device: int = 0):
    buf = C.create_string_buffer(256)
    ok = lib().fp8ln_check_support(device, buf, len(buf))
    return ok == 1, buf.value.decode()


def workspace_size(op: int, a: int, b: int, c: int = 0) -> int:
    return int(lib().fp8ln_workspace_size(op, a, b, c))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ---- delayed-scaling state ----------------------------------------------------

def meta_init(recipe: Recipe, meta: Meta, stream=None) -> None:
    r, m = recipe.as_c(), meta.as_c()
    check(lib().fp8ln_meta_init(C.byref(r), C.byref(m), _stream(stream)))


def scaling_update(recipe: Recipe, meta: Meta, stream=None) -> None:
    r, m = recipe.as_c(), meta.as_c()
    check(lib().fp8ln_scaling_update(C.byref(r), C.byref(m), _stream(stream)))


def scaling_update_batch(recipe: Recipe, metas, stream=None) -> None:
    """scaling_update of every state block in metas, in one launch per 64."""
    arr = (_abi.MetaStruct * len(metas))(*[m.as_c() for m in metas])
    check(lib().fp8ln_scaling_update_batch(C.byref(recipe.as_c()), arr, len(metas),
                                           _stream(stream)))


# ---- kernels ------------------------------------------------------------------

def ln_cast_amax(recipe: Recipe, x, gamma, beta, fp8_dtype: int, scale, amax_ptr: int, out,
                 out_t=None, mean=None, rstd=None, stream=None) -> None:
    """out = encode(LayerNorm(x) * scale); amax recorded at amax_ptr (a float32
    device address, usually Meta.amax_ptr(slot)); scale is a 1-element float32
    device tensor (or view)."""
    rows, hidden = x.shape
    _need(x, torch.bfloat16, (rows, hidden), "x")
    _need(gamma, torch.bfloat16, (hidden,), "gamma")
    _need(beta, torch.bfloat16, (hidden,), "beta")
    _need(out, torch.uint8, (rows, hidden), "out")
    _opt(out_t, torch.uint8, (hidden, rows), "out_t")
    _opt(mean, torch.float32, (rows,), "mean")
    _opt(rstd, torch.float32, (rows,), "rstd")
    r = recipe.as_c()
    check(lib().fp8ln_ln_cast_amax(C.byref(r), rows, hidden, DTYPE_BF16, _ptr(x), _ptr(gamma),
                                   _ptr(beta), fp8_dtype, _ptr(scale), C.c_void_p(amax_ptr),
                                   _ptr(out), _ptr(out_t), _ptr(mean), _ptr(rstd),
                                   _stream(stream)))


def cast_amax(x, fp8_dtype: int, scale, amax_ptr: int, out, out_t=None, colsum=None,
              stream=None) -> None:
    rows, cols = x.shape
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bf16 or float32")
    _need(out, torch.uint8, (rows, cols), "out")
    _opt(out_t, torch.uint8, (cols, rows), "out_t")
    _opt(colsum, torch.float32, (cols,), "colsum")
    ws = None
    nbytes = 0
    if colsum is not None:
        nbytes = workspace_size(_abi.OP_CAST_AMAX, rows, cols)
        ws = _workspace(nbytes, x.device)
    dt = DTYPE_F32 if x.dtype == torch.float32 else DTYPE_BF16
    check(lib().fp8ln_cast_amax(rows, cols, dt, _ptr(x), fp8_dtype, _ptr(scale),
                                C.c_void_p(amax_ptr), _ptr(out), _ptr(out_t), _ptr(colsum),
                                _ptr(ws), nbytes, _stream(stream)))


def stream_probe(x, out, stream=None) -> None:
    """out[i] = high byte of bf16 x[i] (the LayerNorm + cast step's traffic)."""
    if x.dtype != torch.bfloat16 or out.dtype != torch.uint8 or out.numel() != x.numel():
        raise ValueError("x must be bf16 and out uint8 with as many elements")
    check(lib().fp8ln_stream_probe(x.numel(), _ptr(x), _ptr(out), _stream(stream)))


def encode_range(start: int, count: int, fp8_dtype: int, out, stream=None) -> None:
    if out.dtype != torch.uint8 or out.numel() < count:
        raise ValueError("out must be a uint8 tensor with at least count elements")
    check(lib().fp8ln_encode_range(start & 0xFFFFFFFF, count, fp8_dtype, _ptr(out),
                                   _stream(stream)))


def gemm(a, a_dtype: int, b, b_dtype: int, sinv_a, sinv_b, out, bias=None, stream=None) -> None:
    """out[m][n] = (sum_k a[m][k] b[n][k]) * sinv_a * sinv_b (+ bias[n])."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(b, torch.uint8, (N, K), "b")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bf16 or float32")
    _need(out, out.dtype, (M, N), "out")
    _opt(bias, torch.bfloat16, (N,), "bias")
    od = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    check(lib().fp8ln_gemm(M, N, K, _ptr(a), a_dtype, _ptr(b), b_dtype, _ptr(sinv_a),
                           _ptr(sinv_b), _ptr(bias), od, _ptr(out), _stream(stream)))


def gemm_gelu_fp8(a, a_dtype: int, b, b_dtype: int, sinv_a, sinv_b, q_dtype: int, q_scale,
                  q_amax_ptr: int, q_out, q_out_t=None, h_out=None, bias=None,
                  activation: int = GELU_TANH, stream=None):
    """fc1 with the GELU epilogue: h = a.b^T * sinv_a * sinv_b + bias (fp32), h_out =
    bf16(h), q_out = encode(gelu(h) * q_scale), amax of gelu(h) at q_amax_ptr."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(b, torch.uint8, (N, K), "b")
    _need(q_out, torch.uint8, (M, N), "q_out")
    _opt(q_out_t, torch.uint8, (N, M), "q_out_t")
    _opt(h_out, torch.bfloat16, (M, N), "h_out")
    _opt(bias, torch.bfloat16, (N,), "bias")
    check(lib().fp8ln_gemm_gelu_fp8(M, N, K, _ptr(a), a_dtype, _ptr(b), b_dtype, _ptr(sinv_a),
                                    _ptr(sinv_b), _ptr(bias), _ptr(h_out), _ptr(q_out),
                                    _ptr(q_out_t), q_dtype, _ptr(q_scale),
                                    C.c_void_p(q_amax_ptr), activation, _stream(stream)))


def gemm_dgelu(a, a_dtype: int, b, b_dtype: int, sinv_a, sinv_b, h, out,
               activation: int = GELU_TANH, stream=None):
    """out = a.b^T * sinv_a * sinv_b * gelu'(h) (fp32)."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(b, torch.uint8, (N, K), "b")
    _need(h, torch.bfloat16, (M, N), "h")
    _need(out, torch.float32, (M, N), "out")
    check(lib().fp8ln_gemm_dgelu(M, N, K, _ptr(a), a_dtype, _ptr(b), b_dtype, _ptr(sinv_a),
                                 _ptr(sinv_b), _ptr(h), _ptr(out), activation, _stream(stream)))


def gemm_dgelu_fp8(a, a_dtype: int, b, b_dtype: int, sinv_a, sinv_b, h, q_dtype: int, q_scale,
                   q_amax_ptr: int, q_out, q_out_t=None, dbias=None, activation: int = GELU_TANH,
                   stream=None, workspace=None):
    """d = a.b^T * sinv_a * sinv_b * gelu'(h) (fp32, not stored); q_out = encode(d *
    q_scale), q_out_t its transpose, amax of d at q_amax_ptr, dbias = column sums of d."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.uint8, (M, K), "a")
    _need(b, torch.uint8, (N, K), "b")
    _need(h, torch.bfloat16, (M, N), "h")
    _need(q_out, torch.uint8, (M, N), "q_out")
    _opt(q_out_t, torch.uint8, (N, M), "q_out_t")
    _opt(dbias, torch.float32, (N,), "dbias")
    nbytes = workspace_size(OP_GEMM_DGELU_FP8, M, N) if dbias is not None else 0
    ws = None
    if dbias is not None:
        ws = workspace if workspace is not None else _workspace(nbytes, a.device)
        nbytes = ws.numel()
    check(lib().fp8ln_gemm_dgelu_fp8(M, N, K, _ptr(a), a_dtype, _ptr(b), b_dtype, _ptr(sinv_a),
                                     _ptr(sinv_b), _ptr(h), q_dtype, _ptr(q_scale),
                                     C.c_void_p(q_amax_ptr), _ptr(q_out), _ptr(q_out_t),
                                     _ptr(dbias), activation, _ptr(ws), nbytes, _stream(stream)))


def layernorm_bwd(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, stream=None) -> None:
    rows, hidden = x.shape
    _need(dy, torch.float32, (rows, hidden), "dy")
    _need(x, torch.bfloat16, (rows, hidden), "x")
    _need(dx, torch.bfloat16, (rows, hidden), "dx")
    nbytes = workspace_size(_abi.OP_LAYERNORM_BWD, rows, hidden)
    ws = _workspace(nbytes, x.device)
    check(lib().fp8ln_layernorm_bwd(rows, hidden, _ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd),
                                    _ptr(gamma), _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(ws),
                                    nbytes, _stream(stream)))


def layernorm_fwd(x, gamma, beta, y, mean=None, rstd=None, eps=1e-5, stream=None) -> None:
    """The plain LayerNorm module's forward: y = LN(x) in bf16."""
    M, H = x.shape
    _need(x, torch.bfloat16, (M, H), "x")
    _need(y, torch.bfloat16, (M, H), "y")
    _need(gamma, torch.bfloat16, (H,), "gamma")
    _need(beta, torch.bfloat16, (H,), "beta")
    _opt(mean, torch.float32, (M,), "mean")
    _opt(rstd, torch.float32, (M,), "rstd")
    check(lib().fp8ln_layernorm_fwd(M, H, float(eps), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y),
                                    _ptr(mean), _ptr(rstd), _stream(stream)))


def layernorm_bwd_bf16(dy, x, mean, rstd, gamma, dx, dgamma, dbeta, stream=None) -> None:
    """The plain LayerNorm module's backward, for a bf16 incoming gradient."""
    M, H = x.shape
    _need(dy, torch.bfloat16, (M, H), "dy")
    _need(dx, torch.bfloat16, (M, H), "dx")
    ws = _workspace(workspace_size(OP_LAYERNORM_BWD, M, H), x.device)
    check(lib().fp8ln_layernorm_bwd_bf16(M, H, _ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd),
                                         _ptr(gamma), _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                                         _ptr(ws), ws.numel(), _stream(stream)))


# ---- BF16 path (no FP8) ---------------------------------------------------------

def gemm_bf16(a, b, out, bias=None, stream=None) -> None:
    """out = a . b^T (+ bias) with bf16 operands; out bf16, or fp32 without bias."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.bfloat16, (M, K), "a")
    _need(b, torch.bfloat16, (N, K), "b")
    _opt(bias, torch.bfloat16, (N,), "bias")
    odt = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    _need(out, out.dtype, (M, N), "out")
    check(lib().fp8ln_gemm_bf16(M, N, K, _ptr(a), _ptr(b), _ptr(bias), odt, _ptr(out),
                                _stream(stream)))


def gemm_gelu_bf16(a, b, out, bias=None, h_out=None, activation=GELU_TANH, stream=None) -> None:
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.bfloat16, (M, K), "a")
    _need(b, torch.bfloat16, (N, K), "b")
    _opt(bias, torch.bfloat16, (N,), "bias")
    _need(out, torch.bfloat16, (M, N), "out")
    _opt(h_out, torch.bfloat16, (M, N), "h_out")
    check(lib().fp8ln_gemm_gelu_bf16(M, N, K, _ptr(a), _ptr(b), _ptr(bias), _ptr(h_out),
                                     _ptr(out), int(activation), _stream(stream)))


def gemm_dgelu_bf16(a, b, h, out, activation=GELU_TANH, stream=None) -> None:
    """out = bf16((a . b^T) * gelu'(h)) with bf16 operands."""
    M, K = a.shape
    N = b.shape[0]
    _need(a, torch.bfloat16, (M, K), "a")
    _need(b, torch.bfloat16, (N, K), "b")
    _need(h, torch.bfloat16, (M, N), "h")
    _need(out, torch.bfloat16, (M, N), "out")
    check(lib().fp8ln_gemm_dgelu_bf16(M, N, K, _ptr(a), _ptr(b), _ptr(h), _ptr(out),
                                      int(activation), _stream(stream)))


def transpose_bf16(x, out, colsum=None, stream=None) -> None:
    R, Cc = x.shape
    _need(x, torch.bfloat16, (R, Cc), "x")
    _need(out, torch.bfloat16, (Cc, R), "out")
    _opt(colsum, torch.float32, (Cc,), "colsum")
    ws = _workspace(workspace_size(_abi.OP_TRANSPOSE_BF16, R, Cc), x.device)
    check(lib().fp8ln_transpose_bf16(R, Cc, _ptr(x), _ptr(out), _ptr(colsum), _ptr(ws),
                                     ws.numel(), _stream(stream)))


def ln_linear_fwd_bf16(x, gamma, beta, weight, bias, out, ln_out, mean=None, rstd=None,
                       eps=1e-5, stream=None) -> None:
    M, K = x.shape
    N = weight.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(weight, torch.bfloat16, (N, K), "weight")
    _opt(bias, torch.bfloat16, (N,), "bias")
    _need(out, torch.bfloat16, (M, N), "out")
    _need(ln_out, torch.bfloat16, (M, K), "ln_out")
    check(lib().fp8ln_ln_linear_fwd_bf16(M, K, N, float(eps), _ptr(x), _ptr(gamma), _ptr(beta),
                                         _ptr(weight), _ptr(bias), _ptr(out), _ptr(ln_out),
                                         _ptr(mean), _ptr(rstd), _stream(stream)))


def ln_linear_bwd_bf16(dy, x, gamma, weight, ln_out, mean, rstd, dx, dgamma, dbeta, dweight,
                       dbias=None, workspace=None, stream=None) -> None:
    M, N = dy.shape
    K = x.shape[1]
    _need(dy, torch.bfloat16, (M, N), "dy")
    _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dweight, torch.float32, (N, K), "dweight")
    _opt(dbias, torch.float32, (N,), "dbias")
    nbytes = workspace_size(_abi.OP_LN_LINEAR_BWD_BF16, M, K, N)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    check(lib().fp8ln_ln_linear_bwd_bf16(M, K, N, _ptr(dy), _ptr(x), _ptr(gamma), _ptr(weight),
                                         _ptr(ln_out), _ptr(mean), _ptr(rstd), _ptr(dx),
                                         _ptr(dgamma), _ptr(dbeta), _ptr(dweight), _ptr(dbias),
                                         _ptr(workspace), workspace.numel(), _stream(stream)))


def ln_mlp_fwd_bf16(x, gamma, beta, w1, b1, w2, b2, out, ln_out, g, h=None, mean=None,
                    rstd=None, eps=1e-5, activation=GELU_TANH, stream=None) -> None:
    M, H = x.shape
    F = w1.shape[0]
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w1, torch.bfloat16, (F, H), "w1")
    _need(w2, torch.bfloat16, (H, F), "w2")
    _opt(b1, torch.bfloat16, (F,), "b1")
    _opt(b2, torch.bfloat16, (H,), "b2")
    _need(out, torch.bfloat16, (M, H), "out")
    _need(ln_out, torch.bfloat16, (M, H), "ln_out")
    _need(g, torch.bfloat16, (M, F), "g")
    _opt(h, torch.bfloat16, (M, F), "h")
    check(lib().fp8ln_ln_mlp_fwd_bf16(M, H, F, float(eps), int(activation), _ptr(x), _ptr(gamma),
                                      _ptr(beta), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                      _ptr(out), _ptr(ln_out), _ptr(h), _ptr(g), _ptr(mean),
                                      _ptr(rstd), _stream(stream)))


def ln_mlp_bwd_bf16(dy, x, gamma, w1, w2, ln_out, h, g, mean, rstd, dx, dgamma, dbeta, dw1,
                    db1, dw2, db2, activation=GELU_TANH, workspace=None, stream=None) -> None:
    M, H = dy.shape
    F = w1.shape[0]
    _need(dy, torch.bfloat16, (M, H), "dy")
    _need(h, torch.bfloat16, (M, F), "h")
    _need(g, torch.bfloat16, (M, F), "g")
    _need(dx, torch.bfloat16, (M, H), "dx")
    _need(dw1, torch.float32, (F, H), "dw1")
    _need(dw2, torch.float32, (H, F), "dw2")
    _opt(db1, torch.float32, (F,), "db1")
    _opt(db2, torch.float32, (H,), "db2")
    nbytes = workspace_size(_abi.OP_LN_MLP_BWD_BF16, M, H, F)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    check(lib().fp8ln_ln_mlp_bwd_bf16(M, H, F, int(activation), _ptr(dy), _ptr(x), _ptr(gamma),
                                      _ptr(w1), _ptr(w2), _ptr(ln_out), _ptr(h), _ptr(g),
                                      _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dgamma),
                                      _ptr(dbeta), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))


# ---- modules ------------------------------------------------------------------

def linear_fwd(recipe: Recipe, x, weight, bias, out, fwd: Meta, ctx: LinearCtx,
               stream=None) -> None:
    M, K = x.shape
    N = weight.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(weight, torch.bfloat16, (N, K), "weight")
    _opt(bias, torch.bfloat16, (N,), "bias")
    _need(out, torch.bfloat16, (M, N), "out")
    r, m, c = recipe.as_c(), fwd.as_c(), ctx.as_c()
    check(lib().fp8ln_linear_fwd(C.byref(r), M, K, N, DTYPE_BF16, _ptr(x), _ptr(weight),
                                 _ptr(bias), _ptr(out), C.byref(m), C.byref(c), _stream(stream)))


def linear_bwd(recipe: Recipe, dy, ctx: LinearCtx, fwd: Meta, bwd: Meta, dx, dweight,
               dbias=None, workspace=None, stream=None) -> None:
    M, N = dy.shape
    K = dx.shape[1]
    _need(dy, torch.bfloat16, (M, N), "dy")
    _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dweight, torch.float32, (N, K), "dweight")
    _opt(dbias, torch.float32, (N,), "dbias")
    nbytes = workspace_size(OP_LINEAR_BWD, M, K, N)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_linear_bwd(C.byref(r), M, K, N, DTYPE_BF16, _ptr(dy), C.byref(c),
                                 C.byref(mf), C.byref(mb), _ptr(dx), _ptr(dweight), _ptr(dbias),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def step_workspace(device="cuda"):
    """A zeroed step workspace for the *_step calls (every call leaves it zero
    again; one per stream of steps)."""
    return torch.zeros(_abi.STEP_WS_BYTES // 4, dtype=torch.int32, device=device)


def ln_linear_fwd_step(recipe: Recipe, x, gamma, beta, weight, bias, out, fwd: Meta,
                       ctx: LinearCtx, step_ws, stream=None) -> None:
    """scaling_update(recipe, fwd) then ln_linear_fwd(...), the update folded into
    the forward's first launch where the shape allows."""
    M, K = x.shape
    N = weight.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(weight, torch.bfloat16, (N, K), "weight")
    _opt(bias, torch.bfloat16, (N,), "bias")
    _need(out, torch.bfloat16, (M, N), "out")
    _need(step_ws, torch.int32, (_abi.STEP_WS_BYTES // 4,), "step_ws")
    r, m, c = recipe.as_c(), fwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_linear_fwd_step(C.byref(r), M, K, N, DTYPE_BF16, _ptr(x), _ptr(gamma),
                                         _ptr(beta), _ptr(weight), _ptr(bias), _ptr(out),
                                         C.byref(m), C.byref(c), _ptr(step_ws), _stream(stream)))


def ln_linear_fwd(recipe: Recipe, x, gamma, beta, weight, bias, out, fwd: Meta, ctx: LinearCtx,
                  stream=None) -> None:
    M, K = x.shape
    N = weight.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(weight, torch.bfloat16, (N, K), "weight")
    _opt(bias, torch.bfloat16, (N,), "bias")
    _need(out, torch.bfloat16, (M, N), "out")
    r, m, c = recipe.as_c(), fwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_linear_fwd(C.byref(r), M, K, N, DTYPE_BF16, _ptr(x), _ptr(gamma),
                                    _ptr(beta), _ptr(weight), _ptr(bias), _ptr(out), C.byref(m),
                                    C.byref(c), _stream(stream)))


def ln_linear_bwd(recipe: Recipe, dy, x, gamma, ctx: LinearCtx, fwd: Meta, bwd: Meta, dx,
                  dgamma, dbeta, dweight, dbias=None, workspace=None, stream=None) -> None:
    M, N = dy.shape
    K = x.shape[1]
    _need(dy, torch.bfloat16, (M, N), "dy")
    _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dweight, torch.float32, (N, K), "dweight")
    _opt(dbias, torch.float32, (N,), "dbias")
    nbytes = workspace_size(_abi.OP_LN_LINEAR_BWD, M, K, N)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_linear_bwd(C.byref(r), M, K, N, DTYPE_BF16, _ptr(dy), _ptr(x),
                                    _ptr(gamma), C.byref(c), C.byref(mf), C.byref(mb), _ptr(dx),
                                    _ptr(dgamma), _ptr(dbeta), _ptr(dweight), _ptr(dbias),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def ln_linear_bwd_step(recipe: Recipe, dy, x, gamma, ctx: LinearCtx, fwd: Meta, bwd: Meta, dx,
                       dgamma, dbeta, dweight, step_ws, dbias=None, workspace=None,
                       stream=None) -> None:
    """scaling_update(recipe, bwd) then ln_linear_bwd(...), the update folded into
    the gradient cast where it can be."""
    M, N = dy.shape
    K = x.shape[1]
    _need(dy, torch.bfloat16, (M, N), "dy")
    _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dweight, torch.float32, (N, K), "dweight")
    _opt(dbias, torch.float32, (N,), "dbias")
    _need(step_ws, torch.int32, (_abi.STEP_WS_BYTES // 4,), "step_ws")
    nbytes = workspace_size(_abi.OP_LN_LINEAR_BWD, M, K, N)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_linear_bwd_step(C.byref(r), M, K, N, DTYPE_BF16, _ptr(dy), _ptr(x),
                                         _ptr(gamma), C.byref(c), C.byref(mf), C.byref(mb),
                                         _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dweight),
                                         _ptr(dbias), _ptr(workspace), workspace.numel(),
                                         _ptr(step_ws), _stream(stream)))


def ln_linear_bwd_noalloc(recipe: Recipe, dy, x, gamma, ctx: LinearCtx, fwd: Meta, bwd: Meta,
                          dx, dgamma, dbeta, dweight, dbias=None, stream=None) -> None:
    """ln_linear_bwd with its workspace in the library's own device array (no
    allocation by the library or by this binding)."""
    M, N = dy.shape
    K = x.shape[1]
    _need(dy, torch.bfloat16, (M, N), "dy")
    _need(dx, torch.bfloat16, (M, K), "dx")
    _need(dweight, torch.float32, (N, K), "dweight")
    _opt(dbias, torch.float32, (N,), "dbias")
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_linear_bwd_noalloc(C.byref(r), M, K, N, DTYPE_BF16, _ptr(dy), _ptr(x),
                                            _ptr(gamma), C.byref(c), C.byref(mf), C.byref(mb),
                                            _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(dweight),
                                            _ptr(dbias), _stream(stream)))


def ln_mlp_fwd(recipe: Recipe, x, gamma, beta, w1, b1, w2, b2, out, fwd: Meta, ctx: MlpCtx,
               stream=None) -> None:
    M, H = x.shape
    F = w1.shape[0]
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w1, torch.bfloat16, (F, H), "w1")
    _need(w2, torch.bfloat16, (H, F), "w2")
    _opt(b1, torch.bfloat16, (F,), "b1")
    _opt(b2, torch.bfloat16, (H,), "b2")
    _need(out, torch.bfloat16, (M, H), "out")
    r, m, c = recipe.as_c(), fwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_mlp_fwd(C.byref(r), M, H, F, DTYPE_BF16, _ptr(x), _ptr(gamma),
                                 _ptr(beta), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out),
                                 C.byref(m), C.byref(c), _stream(stream)))


def ln_mlp_fwd_step(recipe: Recipe, x, gamma, beta, w1, b1, w2, b2, out, fwd: Meta,
                    ctx: MlpCtx, step_ws, stream=None) -> None:
    """scaling_update(recipe, fwd) then ln_mlp_fwd(...), the update folded into the
    forward's launches where the shape allows."""
    M, H = x.shape
    F = w1.shape[0]
    _need(x, torch.bfloat16, (M, H), "x")
    _need(w1, torch.bfloat16, (F, H), "w1")
    _need(w2, torch.bfloat16, (H, F), "w2")
    _opt(b1, torch.bfloat16, (F,), "b1")
    _opt(b2, torch.bfloat16, (H,), "b2")
    _need(out, torch.bfloat16, (M, H), "out")
    _need(step_ws, torch.int32, (_abi.STEP_WS_BYTES // 4,), "step_ws")
    r, m, c = recipe.as_c(), fwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_mlp_fwd_step(C.byref(r), M, H, F, DTYPE_BF16, _ptr(x), _ptr(gamma),
                                      _ptr(beta), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                      _ptr(out), C.byref(m), C.byref(c), _ptr(step_ws),
                                      _stream(stream)))


def ln_mlp_bwd(recipe: Recipe, dy, x, gamma, ctx: MlpCtx, fwd: Meta, bwd: Meta, dx, dgamma,
               dbeta, dw1, db1, dw2, db2, workspace=None, stream=None) -> None:
    M, H = dy.shape
    F = ctx.w1_q.shape[0]
    _need(dy, torch.bfloat16, (M, H), "dy")
    _need(dx, torch.bfloat16, (M, H), "dx")
    _need(dw1, torch.float32, (F, H), "dw1")
    _need(dw2, torch.float32, (H, F), "dw2")
    _opt(db1, torch.float32, (F,), "db1")
    _opt(db2, torch.float32, (H,), "db2")
    nbytes = workspace_size(_abi.OP_LN_MLP_BWD, M, H, F)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_mlp_bwd(C.byref(r), M, H, F, DTYPE_BF16, _ptr(dy), _ptr(x), _ptr(gamma),
                                 C.byref(c), C.byref(mf), C.byref(mb), _ptr(dx), _ptr(dgamma),
                                 _ptr(dbeta), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def ln_mlp_bwd_step(recipe: Recipe, dy, x, gamma, ctx: MlpCtx, fwd: Meta, bwd: Meta, dx, dgamma,
                    dbeta, dw1, db1, dw2, db2, step_ws, workspace=None, stream=None) -> None:
    """scaling_update(recipe, bwd) then ln_mlp_bwd(...), the update folded into the
    gradient cast where it can be."""
    M, H = dy.shape
    F = ctx.w1_q.shape[0]
    _need(dy, torch.bfloat16, (M, H), "dy")
    _need(dx, torch.bfloat16, (M, H), "dx")
    _need(dw1, torch.float32, (F, H), "dw1")
    _need(dw2, torch.float32, (H, F), "dw2")
    _opt(db1, torch.float32, (F,), "db1")
    _opt(db2, torch.float32, (H,), "db2")
    _need(step_ws, torch.int32, (_abi.STEP_WS_BYTES // 4,), "step_ws")
    nbytes = workspace_size(_abi.OP_LN_MLP_BWD, M, H, F)
    if workspace is None:
        workspace = _workspace(nbytes, dy.device)
    r, mf, mb, c = recipe.as_c(), fwd.as_c(), bwd.as_c(), ctx.as_c()
    check(lib().fp8ln_ln_mlp_bwd_step(C.byref(r), M, H, F, DTYPE_BF16, _ptr(dy), _ptr(x),
                                      _ptr(gamma), C.byref(c), C.byref(mf), C.byref(mb), _ptr(dx),
                                      _ptr(dgamma), _ptr(dbeta), _ptr(dw1), _ptr(db1), _ptr(dw2),
                                      _ptr(db2), _ptr(workspace), workspace.numel(),
                                      _ptr(step_ws), _stream(stream)))


def linear_metas(recipe: Recipe, device="cuda"):
    """Fresh forward (2 slots) and backward (1 slot) state of a LayerNormLinear or
    a Linear."""
    return (Meta(recipe, 2, META_FORWARD, device), Meta(recipe, 1, META_BACKWARD, device))


def mlp_metas(recipe: Recipe, device="cuda"):
    """Fresh forward (4 slots) and backward (2 slots) state of a LayerNormMLP."""
    return (Meta(recipe, 4, META_FORWARD, device), Meta(recipe, 2, META_BACKWARD, device))
