"""CPU oracle for the FP8 delayed-scaling LayerNormLinear / LayerNormMLP path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this package.  The HIP library
never calls it, and it never calls the HIP library: the two share no code.

It is a plain, slow, obviously checkable implementation in float64 (numpy),
written from the method as the pages describe it:

* "Accelerating Transformer Training with NVIDIA Transformer Engine, Fused
  Kernels, BF16, FP8, and GPU Benchmarking" (the tutorial): fused
  LayerNormLinear(H, 3H) and LayerNormMLP(H, 4H) modules with bf16 params
  (setup listing, module tour), a DelayedScaling recipe with format HYBRID,
  amax_history_len 16 and amax_compute_algo "max" (setup listing), variants
  Format.E4M3 and amax_history_len 1024 (generation listing, "things to try"),
  and the per-module state fp8_meta["scaling_fwd"] holding a per-tensor scale
  vector and a 2-D amax history whose row 0 is the most recent (benchmark
  listing, FP8 state inspection).
* "Turbo-charging your transformer training: a hands-on guide": LayerNormMLP is
  layer norm plus two linear layers with GELU ("The building blocks"); delayed
  scaling tracks the amax of each tensor and rescales it on the fly, HYBRID
  mixes E4M3 and E5M2 ("Playing with lower-precision formats: BF16 vs FP8");
  autocast converts activations to FP8 with the scaling and hands gradients
  back in BF16/FP32.

Where the pages are silent the oracle takes a stated reading; each module's
docstring names the readings it depends on.

oracle.cxx is a second implementation of the same steps in plain C++17
(oracle/cpp/fp8ln_oracle.cpp: table-exact FP8 codec, float64 LayerNorm, exact
integer-accumulated FP8 GEMM, binary32 delayed-scaling bookkeeping and the
module chains), with OpenMP over rows; it is pinned on its own and against this
one, and is the one the benchmark times on the host cores.
"""
from .codec import (E4M3, E5M2, FP8_MAX, bf16_to_f64, f64_to_bf16_bits, fp8_decode,
                    fp8_decode_table, fp8_encode, fp8_positive_values)
from .scaling import Meta, fp8_max_for, scaling_update
from .layernorm import layernorm_fwd, layernorm_bwd
from .gelu import gelu_erf, gelu_erf_grad, gelu_tanh, gelu_tanh_grad
from .gemm import fp8_gemm_tn
from .bf16_path import (gemm_bf16, ln_linear_fwd_bf16, ln_linear_bwd_bf16, ln_mlp_fwd_bf16,
                        ln_mlp_bwd_bf16)
from .modules import (Recipe, FORMAT_E4M3, FORMAT_HYBRID, FORMAT_E5M2, GELU_ERF, GELU_TANH,
                      cast_amax,
                      ln_cast_amax, layernorm, linear_fwd, linear_bwd, ln_linear_fwd, ln_linear_bwd, ln_mlp_fwd, ln_mlp_bwd,
                      fwd_format, bwd_format, linear_fwd_meta, linear_bwd_meta,
                      mlp_fwd_meta, mlp_bwd_meta)

__all__ = [
    "E4M3", "E5M2", "FP8_MAX", "bf16_to_f64", "f64_to_bf16_bits", "fp8_decode",
    "fp8_decode_table", "fp8_encode", "fp8_positive_values", "Meta", "fp8_max_for",
    "scaling_update", "layernorm_fwd", "layernorm_bwd", "gelu_tanh", "gelu_tanh_grad",
    "gelu_erf", "gelu_erf_grad", "GELU_TANH", "GELU_ERF",
    "fp8_gemm_tn", "gemm_bf16", "ln_linear_fwd_bf16", "ln_linear_bwd_bf16",
    "ln_mlp_fwd_bf16", "ln_mlp_bwd_bf16", "Recipe", "FORMAT_E4M3", "FORMAT_HYBRID", "FORMAT_E5M2", "cast_amax",
    "ln_cast_amax", "layernorm", "linear_fwd", "linear_bwd", "ln_linear_fwd", "ln_linear_bwd", "ln_mlp_fwd", "ln_mlp_bwd",
    "fwd_format", "bwd_format", "linear_fwd_meta", "linear_bwd_meta", "mlp_fwd_meta",
    "mlp_bwd_meta",
]
