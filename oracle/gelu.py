"""GELU and its derivative in float64 (oracle, test infrastructure only).

LayerNormMLP is layer norm, two linear layers and a GELU ("Turbo-charging ...",
"The building blocks").  The pages do not say which GELU the fused module
uses (the tutorial's plain-PyTorch mirror uses nn.GELU()); this path takes the
tanh approximation:
    gelu(h) = 0.5 h (1 + tanh(u)),  u = sqrt(2/pi) (h + 0.044715 h^3)
    gelu'(h) = 0.5 (1 + t) + 0.5 h (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 h^2),  t = tanh(u)
as the default, and offers the exact erf form of the mirror's nn.GELU() as the
alternative activation:
    gelu(h) = 0.5 h (1 + erf(h / sqrt 2)),
    gelu'(h) = 0.5 (1 + erf(h / sqrt 2)) + h exp(-h^2 / 2) / sqrt(2 pi)
(the library's error function, scipy.special.erf, serves as a step).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

_C = math.sqrt(2.0 / math.pi)
_A = 0.044715


def gelu_tanh(h):
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * h * (1.0 + np.tanh(_C * (h + _A * h ** 3)))


def gelu_tanh_grad(h):
    h = np.asarray(h, dtype=np.float64)
    t = np.tanh(_C * (h + _A * h ** 3))
    return 0.5 * (1.0 + t) + 0.5 * h * (1.0 - t * t) * _C * (1.0 + 3.0 * _A * h * h)


def gelu_erf(h):
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * h * (1.0 + _erf(h / math.sqrt(2.0)))


def gelu_erf_grad(h):
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * (1.0 + _erf(h / math.sqrt(2.0))) + h * np.exp(-0.5 * h * h) / math.sqrt(2.0 * math.pi)
