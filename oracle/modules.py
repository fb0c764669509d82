"""The fused modules' forward and backward chains (oracle, test infrastructure only).

Each function takes the step's inputs as bf16 bit patterns (uint16 arrays),
the recipe and the module's FP8 state (oracle.Meta, mutated in place: the
step's amaxes are recorded into history row 0) and returns float64 results
plus the FP8 codes the step produced.  The caller runs scaling_update on each
Meta at the start of a step, as the delayed-scaling recipe does.

Readings (the pages name the modules and the recipe, not their internals):

* Formats: HYBRID uses E4M3 for forward tensors (activations, weights) and
  E5M2 for gradients ("mixes E4M3 and E5M2", "Turbo-charging ...", "Playing
  with lower-precision formats"); Format.E4M3 (tutorial, "things to try")
  uses E4M3 for both; Format.E5M2 uses E5M2 for both.
* Tensors with FP8 state: LayerNormLinear forward {0: LN output, 1: weight},
  backward {0: output gradient}.  LayerNormMLP forward {0: LN output,
  1: fc1 weight, 2: GELU output (fc2 input), 3: fc2 weight}, backward
  {0: fc2 output gradient, 1: fc1 output gradient}.
* amax is the largest |value| of the tensor before scaling, rounded to
  binary32; q = encode(value * scale) with the slot's binary32 scale.
* The GEMM epilogue is acc * scale_inv_a * scale_inv_b + bias; the MLP applies
  GELU (tanh form by default, erf form as the alternative activation) to fc1's
  output in full precision and casts it to FP8 for
  fc2; fc1's output h is kept as bf16 for the backward's GELU derivative.
* FP8 weight storage ("things to try next": FP8 model init): a forward may
  reuse the FP8 codes an earlier forward made of the unchanged weight, with the
  scale_inv they were made with; such a step records no weight amax.
* Backward: the output gradient is cast to FP8 in the backward format; dgrad
  multiplies it with the forward's FP8 weight codes (and their scale_inv),
  wgrad with the forward's
  FP8 input codes; bias gradients are column sums of the unquantised
  gradient; dx, dgamma, dbeta come from the LayerNorm backward.  Results are
  float64 here; the HIP path returns dx in bf16 and the rest in fp32, the two
  precisions in which the pages have gradients leave FP8 ("Turbo-charging your
  transformer training", "Playing with lower-precision formats: BF16 vs FP8").
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .codec import E4M3, E5M2, bf16_to_f64, f64_to_bf16_bits, fp8_encode
from .gelu import gelu_erf, gelu_erf_grad, gelu_tanh, gelu_tanh_grad

GELU_TANH = 0
GELU_ERF = 1


def _gelu(recipe, h):
    return gelu_erf(h) if recipe.activation == GELU_ERF else gelu_tanh(h)


def _gelu_grad(recipe, h):
    return gelu_erf_grad(h) if recipe.activation == GELU_ERF else gelu_tanh_grad(h)
from .gemm import fp8_gemm_tn
from .layernorm import layernorm_bwd, layernorm_fwd
from .scaling import Meta

FORMAT_E4M3 = 0
FORMAT_HYBRID = 1
FORMAT_E5M2 = 2


@dataclass
class Recipe:
    format: int = FORMAT_HYBRID
    amax_history_len: int = 16
    margin: int = 0
    ln_eps: float = 1e-5
    activation: int = 0          # 0: GELU tanh form, 1: GELU erf form

    @property
    def eps64(self) -> float:
        """The epsilon as the binary32 value the recipe carries."""
        return float(np.float32(self.ln_eps))


def fwd_format(recipe: Recipe) -> str:
    return E5M2 if recipe.format == FORMAT_E5M2 else E4M3


def bwd_format(recipe: Recipe) -> str:
    return E4M3 if recipe.format == FORMAT_E4M3 else E5M2


def linear_fwd_meta(recipe: Recipe) -> Meta:
    return Meta.fresh(recipe.amax_history_len, [fwd_format(recipe)] * 2)


def linear_bwd_meta(recipe: Recipe) -> Meta:
    return Meta.fresh(recipe.amax_history_len, [bwd_format(recipe)])


def mlp_fwd_meta(recipe: Recipe) -> Meta:
    return Meta.fresh(recipe.amax_history_len, [fwd_format(recipe)] * 4)


def mlp_bwd_meta(recipe: Recipe) -> Meta:
    return Meta.fresh(recipe.amax_history_len, [bwd_format(recipe)] * 2)


def _amax(v: np.ndarray) -> np.float32:
    if v.size == 0:
        return np.float32(0.0)
    if np.isnan(v).any():
        return np.float32(np.nan)
    return np.float32(np.abs(v).max())


def cast_amax(values: np.ndarray, scale: np.float32, fmt: str):
    """(codes, amax) for one tensor: codes = encode(values * scale)."""
    v = np.asarray(values, dtype=np.float64)
    q = fp8_encode(v * float(np.float32(scale)), fmt)
    return q, _amax(v)


def ln_cast_amax(x_bits, gamma_bits, beta_bits, eps: float, scale: np.float32, fmt: str):
    """LayerNorm each row, then cast to FP8.  Returns dict(q, amax, y, mean, rstd)."""
    x = bf16_to_f64(x_bits)
    y, mean, rstd = layernorm_fwd(x, bf16_to_f64(gamma_bits), bf16_to_f64(beta_bits), eps)
    q, amax = cast_amax(y, scale, fmt)
    return dict(q=q, amax=amax, y=y, mean=mean, rstd=rstd)


def layernorm(x_bits, gamma_bits, beta_bits, eps: float):
    """The plain LayerNorm module: y = LN(x) rounded once to bf16.  Returns
    dict(y_bits, y, mean, rstd)."""
    y, mean, rstd = layernorm_fwd(bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                  bf16_to_f64(beta_bits), eps)
    return dict(y_bits=f64_to_bf16_bits(y), y=y, mean=mean, rstd=rstd)


def _bias(b_bits, n):
    return np.zeros(n) if b_bits is None else bf16_to_f64(b_bits)


def _weight(meta: Meta, slot: int, w_bits, fmt: str, cached):
    """The weight's FP8 codes and the scale_inv they were made with.  Without a
    cache the weight is cast with the slot's scale and its amax recorded; with
    FP8 weight storage (cached = (codes, scale_inv) of an earlier forward on the
    unchanged weight) the stored codes are used as they are and this step
    records no weight amax."""
    if cached is not None:
        return cached[0], np.float32(cached[1]), None
    w_q, w_amax = cast_amax(bf16_to_f64(w_bits), meta.scale[slot], fmt)
    meta.record_amax(slot, w_amax)
    return w_q, np.float32(meta.scale_inv[slot]), w_amax


def linear_fwd(recipe: Recipe, meta: Meta, x_bits, w_bits, bias_bits=None, cached_w=None):
    """out = x W^T + b with FP8 operands (Linear: no LayerNorm).  Slot 0 is the
    input x itself; the rest is ln_linear_fwd."""
    fmt = fwd_format(recipe)
    x_q, x_amax = cast_amax(bf16_to_f64(x_bits), meta.scale[0], fmt)
    meta.record_amax(0, x_amax)
    w_q, w_sinv, w_amax = _weight(meta, 1, w_bits, fmt, cached_w)
    out = fp8_gemm_tn(x_q, fmt, w_q, fmt, meta.scale_inv[0], w_sinv,
                      _bias(bias_bits, w_q.shape[0]))
    ctx = dict(x_q=x_q, w_q=w_q, w_sinv=w_sinv, x_amax=x_amax, w_amax=w_amax)
    return out, ctx


def linear_bwd(recipe: Recipe, meta_fwd: Meta, meta_bwd: Meta, dy_bits, ctx):
    """Gradients of linear_fwd for dy [M][N]: dx = dy W, dW = dy^T x (both from
    FP8 codes), dbias = column sums of dy."""
    ffmt, bfmt = fwd_format(recipe), bwd_format(recipe)
    dy = bf16_to_f64(dy_bits)
    dy_q, dy_amax = cast_amax(dy, meta_bwd.scale[0], bfmt)
    meta_bwd.record_amax(0, dy_amax)
    dx = fp8_gemm_tn(dy_q, bfmt, ctx["w_q"].T, ffmt, meta_bwd.scale_inv[0], ctx["w_sinv"])
    dw = fp8_gemm_tn(dy_q.T, bfmt, ctx["x_q"].T, ffmt, meta_bwd.scale_inv[0],
                     meta_fwd.scale_inv[0])
    return dict(dx=dx, dw=dw, dbias=dy.sum(axis=0), dy_q=dy_q, dy_amax=dy_amax)


def ln_linear_fwd(recipe: Recipe, meta: Meta, x_bits, gamma_bits, beta_bits, w_bits,
                  bias_bits=None, cached_w=None):
    """out = LN(x) W^T + b with FP8 operands.  x [M][K], W [N][K].  cached_w:
    (w_q, w_sinv) of an earlier forward to reuse (FP8 weight storage)."""
    fmt = fwd_format(recipe)
    ln = ln_cast_amax(x_bits, gamma_bits, beta_bits, recipe.eps64, meta.scale[0], fmt)
    meta.record_amax(0, ln["amax"])
    w_q, w_sinv, w_amax = _weight(meta, 1, w_bits, fmt, cached_w)
    out = fp8_gemm_tn(ln["q"], fmt, w_q, fmt, meta.scale_inv[0], w_sinv,
                      _bias(bias_bits, w_q.shape[0]))
    ctx = dict(ln_q=ln["q"], w_q=w_q, w_sinv=w_sinv, mean=ln["mean"], rstd=ln["rstd"],
               y=ln["y"], ln_amax=ln["amax"], w_amax=w_amax)
    return out, ctx


def ln_linear_bwd(recipe: Recipe, meta_fwd: Meta, meta_bwd: Meta, dy_bits, ctx, x_bits,
                  gamma_bits):
    """Gradients of ln_linear_fwd for the output gradient dy [M][N]."""
    ffmt, bfmt = fwd_format(recipe), bwd_format(recipe)
    dy = bf16_to_f64(dy_bits)
    dy_q, dy_amax = cast_amax(dy, meta_bwd.scale[0], bfmt)
    meta_bwd.record_amax(0, dy_amax)
    dbias = dy.sum(axis=0)
    # dgrad: dLN[m][k] = sum_n dy[m][n] W[n][k]
    dln = fp8_gemm_tn(dy_q, bfmt, ctx["w_q"].T, ffmt, meta_bwd.scale_inv[0], ctx["w_sinv"])
    # wgrad: dW[n][k] = sum_m dy[m][n] LN(x)[m][k]
    dw = fp8_gemm_tn(dy_q.T, bfmt, ctx["ln_q"].T, ffmt, meta_bwd.scale_inv[0],
                     meta_fwd.scale_inv[0])
    dx, dgamma, dbeta = layernorm_bwd(dln, bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                      ctx["mean"], ctx["rstd"])
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw=dw, dbias=dbias, dy_q=dy_q,
                dy_amax=dy_amax, dln=dln)


def ln_mlp_fwd(recipe: Recipe, meta: Meta, x_bits, gamma_bits, beta_bits, w1_bits, b1_bits,
               w2_bits, b2_bits, cached_w=None):
    """out = fc2(GELU(fc1(LN(x)))) with FP8 operands.  W1 [F][H], W2 [H][F].
    cached_w: ((w1_q, w1_sinv), (w2_q, w2_sinv)) of an earlier forward to reuse."""
    fmt = fwd_format(recipe)
    ln = ln_cast_amax(x_bits, gamma_bits, beta_bits, recipe.eps64, meta.scale[0], fmt)
    meta.record_amax(0, ln["amax"])
    c1, c2 = (None, None) if cached_w is None else cached_w
    w1_q, w1_sinv, w1_amax = _weight(meta, 1, w1_bits, fmt, c1)
    w2_q, w2_sinv, w2_amax = _weight(meta, 3, w2_bits, fmt, c2)
    h = fp8_gemm_tn(ln["q"], fmt, w1_q, fmt, meta.scale_inv[0], w1_sinv,
                    _bias(b1_bits, w1_q.shape[0]))
    g = _gelu(recipe, h)
    g_q, g_amax = cast_amax(g, meta.scale[2], fmt)
    meta.record_amax(2, g_amax)
    out = fp8_gemm_tn(g_q, fmt, w2_q, fmt, meta.scale_inv[2], w2_sinv,
                      _bias(b2_bits, w2_q.shape[0]))
    ctx = dict(ln_q=ln["q"], w1_q=w1_q, w2_q=w2_q, w1_sinv=w1_sinv, w2_sinv=w2_sinv, h=h,
               h_bits=f64_to_bf16_bits(h), g=g, g_q=g_q, mean=ln["mean"], rstd=ln["rstd"],
               y=ln["y"], ln_amax=ln["amax"], w1_amax=w1_amax, w2_amax=w2_amax, g_amax=g_amax)
    return out, ctx


def ln_mlp_bwd(recipe: Recipe, meta_fwd: Meta, meta_bwd: Meta, dy_bits, ctx, x_bits,
               gamma_bits):
    """Gradients of ln_mlp_fwd for the output gradient dy [M][H]."""
    ffmt, bfmt = fwd_format(recipe), bwd_format(recipe)
    dy = bf16_to_f64(dy_bits)
    dy_q, dy_amax = cast_amax(dy, meta_bwd.scale[0], bfmt)
    meta_bwd.record_amax(0, dy_amax)
    db2 = dy.sum(axis=0)
    # fc2 dgrad, then the GELU derivative at the saved bf16 h
    dg = fp8_gemm_tn(dy_q, bfmt, ctx["w2_q"].T, ffmt, meta_bwd.scale_inv[0], ctx["w2_sinv"])
    dh = dg * _gelu_grad(recipe, bf16_to_f64(ctx["h_bits"]))
    dh_q, dh_amax = cast_amax(dh, meta_bwd.scale[1], bfmt)
    meta_bwd.record_amax(1, dh_amax)
    db1 = dh.sum(axis=0)
    dw2 = fp8_gemm_tn(dy_q.T, bfmt, ctx["g_q"].T, ffmt, meta_bwd.scale_inv[0],
                      meta_fwd.scale_inv[2])
    dln = fp8_gemm_tn(dh_q, bfmt, ctx["w1_q"].T, ffmt, meta_bwd.scale_inv[1], ctx["w1_sinv"])
    dw1 = fp8_gemm_tn(dh_q.T, bfmt, ctx["ln_q"].T, ffmt, meta_bwd.scale_inv[1],
                      meta_fwd.scale_inv[0])
    dx, dgamma, dbeta = layernorm_bwd(dln, bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                      ctx["mean"], ctx["rstd"])
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw1=dw1, db1=db1, dw2=dw2, db2=db2,
                dy_q=dy_q, dy_amax=dy_amax, dh=dh, dh_q=dh_q, dh_amax=dh_amax, dg=dg, dln=dln)
