"""The C-ABI library loads and exports every entry point include/fp8ln.h declares,
and its host-side checks reject bad arguments before touching a device (CPU)."""
import ctypes as C
import os
import re

import pytest

from fp8_delayed_scaling_row_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "fp8ln.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8ln_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail(f"{_abi.LIB_PATH} is not built (python -m fp8_delayed_scaling_row_amd.build)")
    return _abi.lib()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for required in ("fp8ln_ln_cast_amax", "fp8ln_scaling_update", "fp8ln_ln_linear_fwd",
                     "fp8ln_ln_linear_bwd", "fp8ln_ln_mlp_fwd", "fp8ln_ln_mlp_bwd",
                     "fp8ln_meta_init", "fp8ln_gemm", "fp8ln_cast_amax"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    assert sorted(_abi.SIGNATURES) == declared_functions()


def test_status_strings(lib):
    assert lib.fp8ln_status_string(0) == b"ok"
    assert lib.fp8ln_status_string(-1) == b"invalid argument"
    assert lib.fp8ln_status_string(-2) == b"unsupported"
    assert lib.fp8ln_status_string(-3) == b"HIP error"


def test_workspace_sizes_are_host_only_and_monotone(lib):
    f = lib.fp8ln_workspace_size
    assert f(_abi.OP_LN_LINEAR_BWD, 2048, 768, 2304) > 2048 * 768 * 4
    assert f(_abi.OP_LN_MLP_BWD, 2048, 768, 3072) > f(_abi.OP_LN_LINEAR_BWD, 2048, 768, 2304)
    # one fp32 row of column sums per 128-row tile
    assert f(_abi.OP_CAST_AMAX, 2048, 2304, 0) == 16 * 2304 * 4
    assert f(_abi.OP_CAST_AMAX, 2049, 2304, 0) == 17 * 2304 * 4
    assert f(_abi.OP_GEMM_DGELU_FP8, 2048, 3072, 0) == 16 * 3072 * 4
    assert f(99, 1, 1, 1) == 0 and f(_abi.OP_LN_LINEAR_BWD, 16, 16, 0) == 0


def _recipe(**kw):
    r = dict(format=_abi.FORMAT_HYBRID, amax_history_len=16, margin=0, ln_eps=1e-5,
             activation=_abi.GELU_TANH)
    r.update(kw)
    return _abi.Recipe(r["format"], r["amax_history_len"], r["margin"], r["ln_eps"],
                       r["activation"])


@pytest.mark.parametrize("bad,status", [
    (dict(amax_history_len=0), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(amax_history_len=1025), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(format=7), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(margin=-1), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(ln_eps=0.0), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(ln_eps=float("nan")), _abi.FP8LN_ERR_INVALID_ARG),
    (dict(activation=2), _abi.FP8LN_ERR_INVALID_ARG),
])
def test_bad_recipe_is_rejected_before_any_launch(lib, bad, status):
    r = _recipe(**bad)
    m = _abi.MetaStruct(16, 16, 16, 1, 0)     # never dereferenced
    assert lib.fp8ln_scaling_update(C.byref(r), C.byref(m), None) == status
    assert lib.fp8ln_last_error()


def test_unsupported_shapes_and_dtypes_are_rejected(lib):
    r = _recipe()
    p = C.c_void_p(256)   # never dereferenced: validation fails first
    # hidden not a multiple of 8
    s = lib.fp8ln_ln_cast_amax(C.byref(r), 4, 12, _abi.DTYPE_BF16, p, p, p, 0, p, p, p, None,
                               None, None, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # float32 params are not a supported params_dtype
    s = lib.fp8ln_ln_cast_amax(C.byref(r), 4, 16, _abi.DTYPE_F32, p, p, p, 0, p, p, p, None,
                               None, None, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # GEMM with K not a multiple of 16
    s = lib.fp8ln_gemm(16, 16, 24, p, 0, p, 0, p, p, None, _abi.DTYPE_BF16, p, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # negative sizes
    s = lib.fp8ln_gemm(-1, 16, 16, p, 0, p, 0, p, p, None, _abi.DTYPE_BF16, p, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG
    # backward needs tokens % 16 == 0
    mf = _abi.MetaStruct(256, 256, 256, 2, _abi.META_FORWARD)
    mb = _abi.MetaStruct(256, 256, 256, 1, _abi.META_BACKWARD)
    ctx = _abi.LinearCtxStruct(256, 256, 256, 256, 256, 256)
    s = lib.fp8ln_ln_linear_bwd(C.byref(r), 20, 768, 2304, _abi.DTYPE_BF16, p, p, p,
                                C.byref(ctx), C.byref(mf), C.byref(mb), p, p, p, p, None, p,
                                1 << 30, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # wrong meta kind
    s = lib.fp8ln_ln_linear_bwd(C.byref(r), 32, 768, 2304, _abi.DTYPE_BF16, p, p, p,
                                C.byref(ctx), C.byref(mb), C.byref(mf), p, p, p, p, None, p,
                                1 << 30, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG
    # misaligned pointer
    s = lib.fp8ln_cast_amax(16, 16, _abi.DTYPE_BF16, C.c_void_p(257), 0, p, p, p, None, None,
                            None, 0, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG
    assert b"aligned" in lib.fp8ln_last_error()


def test_forward_step_checks_its_workspace(lib):
    r = _recipe()
    p = C.c_void_p(256)
    mf = _abi.MetaStruct(256, 256, 256, 2, _abi.META_FORWARD)
    ctx = _abi.LinearCtxStruct(256, 256, 256, 256, 256, 256)
    args = (C.byref(r), 32, 768, 2304, _abi.DTYPE_BF16, p, p, p, p, None, p, C.byref(mf),
            C.byref(ctx))
    s = lib.fp8ln_ln_linear_fwd_step(*args, None, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG and b"step_ws" in lib.fp8ln_last_error()
    s = lib.fp8ln_ln_linear_fwd_step(*args, C.c_void_p(260), None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG and b"aligned" in lib.fp8ln_last_error()


def test_backward_steps_check_their_workspace(lib):
    r = _recipe()
    p = C.c_void_p(256)
    mf = _abi.MetaStruct(256, 256, 256, 4, _abi.META_FORWARD)
    mb = _abi.MetaStruct(256, 256, 256, 2, _abi.META_BACKWARD)
    lctx = _abi.LinearCtxStruct(256, 256, 256, 256, 256, 256)
    s = lib.fp8ln_ln_linear_bwd_step(C.byref(r), 32, 768, 2304, _abi.DTYPE_BF16, p, p, p,
                                     C.byref(lctx), C.byref(mf), C.byref(mb), p, p, p, p, None,
                                     p, 1 << 30, None, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG and b"step_ws" in lib.fp8ln_last_error()
    mctx = _abi.MlpCtxStruct(*([256] * len(_abi.MlpCtxStruct._fields_)))
    s = lib.fp8ln_ln_mlp_bwd_step(C.byref(r), 32, 768, 3072, _abi.DTYPE_BF16, p, p, p,
                                  C.byref(mctx), C.byref(mf), C.byref(mb), p, p, p, p, None, p,
                                  None, p, 1 << 30, None, None)
    assert s == _abi.FP8LN_ERR_INVALID_ARG and b"step_ws" in lib.fp8ln_last_error()


def test_check_support_reports_a_reason_without_a_gpu(lib):
    buf = C.create_string_buffer(128)
    ok = lib.fp8ln_check_support(0, buf, len(buf))
    assert ok in (0, 1)
    if ok == 0:
        assert buf.value   # a reason is given


# ---- size limits of the GEMM tiles (checked on the host, before any launch) ----

BIG_K = 1 << 23          # 256 rows of 2^23 bytes reach 2^31: past the 32-bit tile offsets
OK_K = (1 << 23) - 16    # the largest multiple of 16 below the limit


def test_gemm_contraction_length_is_bounded(lib):
    p = C.c_void_p(256)   # never dereferenced
    s = lib.fp8ln_gemm(16, 16, BIG_K, p, 0, p, 0, p, p, None, _abi.DTYPE_F32, p, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    assert b"contraction" in lib.fp8ln_last_error()
    # bf16 operands: K counts elements of 2 bytes
    s = lib.fp8ln_gemm_bf16(16, 16, BIG_K // 2, p, p, None, _abi.DTYPE_F32, p, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # the fused GELU' epilogue reads h rows of N bf16 values
    s = lib.fp8ln_gemm_dgelu(16, BIG_K // 2, 16, p, 0, p, 0, p, p, p, p, 0, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    s = lib.fp8ln_gemm_dgelu_fp8(16, BIG_K // 2, 16, p, 0, p, 0, p, p, p, 1, p, p, p, None,
                                 None, 0, None, 0, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED


def test_gemm_output_tiles_are_bounded(lib):
    p = C.c_void_p(256)
    s = lib.fp8ln_gemm(1 << 20, 1 << 20, 16, p, 0, p, 0, p, p, None, _abi.DTYPE_F32, p, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED


def test_token_count_of_the_weight_gradient_is_bounded(lib):
    """wgrad contracts over tokens: a backward over 2^23 tokens is refused
    before any launch (its workspace is never touched)."""
    r = _recipe()
    p = C.c_void_p(256)
    mf = _abi.MetaStruct(256, 256, 256, 2, _abi.META_FORWARD)
    mb = _abi.MetaStruct(256, 256, 256, 1, _abi.META_BACKWARD)
    ctx = _abi.LinearCtxStruct(256, 256, 256, 256, 256, 256)
    huge = C.c_size_t(-1).value
    s = lib.fp8ln_ln_linear_bwd(C.byref(r), BIG_K, 768, 2304, _abi.DTYPE_BF16, p, p, p,
                                C.byref(ctx), C.byref(mf), C.byref(mb), p, p, p, p, None, p,
                                huge, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    assert b"wgrad" in lib.fp8ln_last_error()
    s = lib.fp8ln_linear_bwd(C.byref(r), BIG_K, 768, 2304, _abi.DTYPE_BF16, p, C.byref(ctx),
                             C.byref(mf), C.byref(mb), p, p, None, p, huge, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    mf4 = _abi.MetaStruct(256, 256, 256, 4, _abi.META_FORWARD)
    mb2 = _abi.MetaStruct(256, 256, 256, 2, _abi.META_BACKWARD)
    mctx = _abi.MlpCtxStruct(*([256] * 11))
    s = lib.fp8ln_ln_mlp_bwd(C.byref(r), BIG_K, 768, 3072, _abi.DTYPE_BF16, p, p, p,
                             C.byref(mctx), C.byref(mf4), C.byref(mb2), p, p, p, p, p, p, p, p,
                             huge, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED
    # the BF16 backward as well (2-byte operands: half the tokens suffice)
    s = lib.fp8ln_ln_linear_bwd_bf16(BIG_K // 2, 768, 2304, p, p, p, p, p, p, p, p, p, p, p,
                                     None, p, huge, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED


def test_transposed_copies_bound_the_rows(lib):
    r = _recipe()
    p = C.c_void_p(256)
    s = lib.fp8ln_ln_cast_amax(C.byref(r), 65536 * 64, 64, _abi.DTYPE_BF16, p, p, p, 0, p, p,
                               p, p, None, None, None)
    assert s == _abi.FP8LN_ERR_UNSUPPORTED


def test_largest_contraction_passes_the_size_check(lib):
    """K just below the limit passes validation: without a GPU the call gets as
    far as the device check (a HIP error or UNSUPPORTED device), never the size
    error."""
    p = C.c_void_p(256)
    lib.fp8ln_gemm(16, 16, OK_K, p, 0, p, 0, p, p, None, _abi.DTYPE_F32, p, None)
    assert b"contraction" not in lib.fp8ln_last_error()


C_CALLER = r"""
#include <stdio.h>
#include "fp8ln.h"
int main(void) {
    char reason[128];
    const int ok = fp8ln_check_support(0, reason, sizeof reason);
    fp8ln_recipe r = {0};
    r.amax_history_len = 0;   /* outside 1..1024: refused before any device call */
    const int s = fp8ln_scaling_update(&r, NULL, NULL);
    printf("%s|%s|%d\n", fp8ln_status_string(FP8LN_OK), fp8ln_status_string(s), ok == 0 || ok == 1);
    return s == FP8LN_ERR_INVALID_ARG ? 0 : 1;
}
"""


def test_header_serves_a_c99_caller(tmp_path):
    """The boundary is plain C: a C99 program (pedantic, warnings as errors)
    includes the header, links the library and calls it (argument checks and
    status strings need no GPU)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail(f"{_abi.LIB_PATH} is not built")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(_abi.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe), f"-L{libdir}",
                    "-lfp8ln", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True,
                   text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok|invalid argument|1", r.stdout
