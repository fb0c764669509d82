"""FP8 delayed-scaling LayerNormLinear / LayerNormMLP for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
include/fp8ln.h (libfp8ln.so, built by `python -m fp8_delayed_scaling_row_amd.build`);
`fp8_delayed_scaling_row_amd.ops` is its Python binding and
`fp8_delayed_scaling_row_amd.inputs` draws seeded synthetic inputs.
"""
__version__ = "0.1.0"
