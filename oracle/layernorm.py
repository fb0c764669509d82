"""LayerNorm forward and backward in float64 (oracle, test infrastructure only).

The fused modules normalise each row before the linear layer (tutorial, setup
listing: te.LayerNormLinear / te.LayerNormMLP; "Turbo-charging ...", "The
building blocks": layer norm fused with the following projection).  The pages
do not give epsilon or the variance estimator; the tutorial's plain-PyTorch
mirror block uses nn.LayerNorm with its defaults, so the reading is: biased
variance, eps = 1e-5 (the recipe's float32 value), y = (x - mean) * rstd *
gamma + beta with rstd = 1 / sqrt(var + eps).

Everything is computed in float64 with a two-pass mean/variance, per row.
"""
from __future__ import annotations

import numpy as np


def layernorm_fwd(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """x [rows][H] float64, gamma/beta [H] float64 -> (y, mean, rstd), float64."""
    x = np.asarray(x, dtype=np.float64)
    H = x.shape[-1]
    mean = x.sum(axis=-1) / H
    d = x - mean[..., None]
    var = (d * d).sum(axis=-1) / H
    rstd = 1.0 / np.sqrt(var + float(eps))
    xhat = d * rstd[..., None]
    y = xhat * gamma + beta
    return y, mean, rstd


def layernorm_bwd(dy: np.ndarray, x: np.ndarray, gamma: np.ndarray, mean: np.ndarray,
                  rstd: np.ndarray):
    """Gradients of y = xhat * gamma + beta with xhat = (x - mean) * rstd.

    With g = dy * gamma (per row, H entries):
        dx = rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))
        dgamma = sum over rows of dy * xhat,  dbeta = sum over rows of dy.
    mean and rstd are the forward's statistics (as saved)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    xhat = (x - mean[..., None]) * rstd[..., None]
    g = dy * gamma
    c1 = g.mean(axis=-1)
    c2 = (g * xhat).mean(axis=-1)
    dx = rstd[..., None] * (g - c1[..., None] - xhat * c2[..., None])
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    return dx, dgamma, dbeta
