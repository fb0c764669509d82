"""FP8 GEMM on decoded values (oracle, test infrastructure only).

The fused modules' linear layers run on FP8 operands ("Turbo-charging ...",
"Playing with lower-precision formats": autocast converts activations to FP8
and applies the scaling; tutorial intro: FP8 tensor cores).  The pages give no
epilogue; the reading is C = (sum_k A[i,k] B[j,k]) * sinv_a * sinv_b (+ bias),
with A and B the FP8 codes decoded exactly.

The contraction is a float64 matrix product of the decoded values (a library
primitive).  Every FP8 value is a short binary fraction, so every product is
exact in float64 and the sum is exact too for the operand ranges this path
produces with E4M3 operands (all terms share the unit 2^-18 and the sum stays
far below 2^53 units); with E5M2 operands the sum carries at most float64
rounding, about 1e-16 relative.
"""
from __future__ import annotations

import numpy as np

from .codec import fp8_decode


def fp8_gemm_tn(a_codes, a_fmt, b_codes, b_fmt, sinv_a=1.0, sinv_b=1.0, bias=None):
    """C[i][j] = sum_k dec(A[i][k]) * dec(B[j][k]) * sinv_a * sinv_b + bias[j].

    A is [M][K], B is [N][K]: both operands keep the contraction index last."""
    a = fp8_decode(a_codes, a_fmt)
    b = fp8_decode(b_codes, b_fmt)
    c = a @ b.T
    c = c * float(np.float32(sinv_a)) * float(np.float32(sinv_b))
    if bias is not None:
        c = c + np.asarray(bias, dtype=np.float64)[None, :]
    return c
