"""The same modules without FP8 (oracle, test infrastructure only).

The pages compare FP8 training against BF16 training of the same model
("Turbo-charging your transformer training", "Playing with lower-precision
formats: BF16 vs FP8"; tutorial "Accelerating Transformer Training ...",
benchmark listing and results).  Without FP8 the modules are plain bf16 layers
with fp32 (here float64) accumulation.  Readings (the pages do not spell out
the BF16 modules' internals):

* The LayerNorm output is rounded once to bf16 and that bf16 tensor is the
  GEMM's input, as a bf16 nn.LayerNorm feeding an nn.Linear would be; the
  backward's weight gradient uses the same bf16 tensor.
* fc1's output h stays in full precision for GELU; g = GELU(h) is rounded to
  bf16 and is fc2's input.  h is also stored in bf16 for the backward, whose
  GELU derivative takes that stored bf16 h (as the FP8 path does).
* Backward: dH = (dy W2) * gelu'(h) is rounded to bf16 (the GEMM input dtype of
  this path) and that bf16 dH feeds fc1's weight gradient, its input gradient
  and db1 (column sums).
* Outputs are returned in float64; the HIP path rounds out and dx to bf16 and
  returns dW, dgamma, dbeta and dbias in fp32.
"""
from __future__ import annotations

import numpy as np

from .codec import bf16_to_f64, f64_to_bf16_bits
from .gelu import gelu_erf, gelu_erf_grad, gelu_tanh, gelu_tanh_grad
from .layernorm import layernorm_bwd, layernorm_fwd

GELU_TANH = 0
GELU_ERF = 1


def gemm_bf16(a_bits, b_bits, bias_bits=None):
    """C[i][j] = sum_k A[i][k] B[j][k] + bias[j] on the bf16 values (A [M][K],
    B [N][K]); each product of two bf16 values is exact in float64."""
    c = bf16_to_f64(a_bits) @ bf16_to_f64(b_bits).T
    if bias_bits is not None:
        c = c + bf16_to_f64(bias_bits)[None, :]
    return c


def ln_linear_fwd_bf16(x_bits, gamma_bits, beta_bits, w_bits, bias_bits, eps: float):
    """out = bf16(LN(x)) . W^T + b.  Returns (out, ctx)."""
    y, mean, rstd = layernorm_fwd(bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                  bf16_to_f64(beta_bits), eps)
    ln_bits = f64_to_bf16_bits(y)
    out = gemm_bf16(ln_bits, w_bits, bias_bits)
    return out, dict(ln_bits=ln_bits, y=y, mean=mean, rstd=rstd)


def ln_linear_bwd_bf16(dy_bits, ctx, x_bits, gamma_bits, w_bits):
    """dLN = dy W, dW = dy^T bf16(LN(x)), dbias = column sums of dy, then the
    LayerNorm backward."""
    dy = bf16_to_f64(dy_bits)
    dln = dy @ bf16_to_f64(w_bits)
    dw = dy.T @ bf16_to_f64(ctx["ln_bits"])
    dx, dgamma, dbeta = layernorm_bwd(dln, bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                      ctx["mean"], ctx["rstd"])
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw=dw, dbias=dy.sum(axis=0), dln=dln)


def ln_mlp_fwd_bf16(x_bits, gamma_bits, beta_bits, w1_bits, b1_bits, w2_bits, b2_bits,
                    eps: float, activation: int = GELU_TANH):
    """out = bf16(GELU(bf16(LN(x)) W1^T + b1)) W2^T + b2.  Returns (out, ctx)."""
    y, mean, rstd = layernorm_fwd(bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                  bf16_to_f64(beta_bits), eps)
    ln_bits = f64_to_bf16_bits(y)
    h = gemm_bf16(ln_bits, w1_bits, b1_bits)
    g = gelu_erf(h) if activation == GELU_ERF else gelu_tanh(h)
    g_bits = f64_to_bf16_bits(g)
    out = gemm_bf16(g_bits, w2_bits, b2_bits)
    return out, dict(ln_bits=ln_bits, h=h, h_bits=f64_to_bf16_bits(h), g=g, g_bits=g_bits,
                     mean=mean, rstd=rstd)


def ln_mlp_bwd_bf16(dy_bits, ctx, x_bits, gamma_bits, w1_bits, w2_bits,
                    activation: int = GELU_TANH):
    """Gradients of ln_mlp_fwd_bf16 for dy [M][H].  ctx needs ln_bits, h_bits
    (the stored bf16 h), g_bits, mean and rstd."""
    dy = bf16_to_f64(dy_bits)
    hb = bf16_to_f64(ctx["h_bits"])
    dw2 = dy.T @ bf16_to_f64(ctx["g_bits"])
    dgelu = gelu_erf_grad(hb) if activation == GELU_ERF else gelu_tanh_grad(hb)
    dh = (dy @ bf16_to_f64(w2_bits)) * dgelu
    dh_bits = f64_to_bf16_bits(dh)
    dhb = bf16_to_f64(dh_bits)
    dw1 = dhb.T @ bf16_to_f64(ctx["ln_bits"])
    dln = dhb @ bf16_to_f64(w1_bits)
    dx, dgamma, dbeta = layernorm_bwd(dln, bf16_to_f64(x_bits), bf16_to_f64(gamma_bits),
                                      ctx["mean"], ctx["rstd"])
    return dict(dx=dx, dgamma=dgamma, dbeta=dbeta, dw1=dw1, db1=dhb.sum(axis=0), dw2=dw2,
                db2=dy.sum(axis=0), dh=dh, dh_bits=dh_bits, dln=dln)
