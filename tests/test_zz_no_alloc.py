"""GPU check of the no-allocation LayerNormLinear backward: through the C-ABI it
gives, bit for bit, what fp8ln_ln_linear_bwd gives with a caller workspace,
on two calls in a row (the second smaller, so it runs over the first call's
leftovers in the library's array)."""
import numpy as np
import pytest
import torch

from fp8_delayed_scaling_row_amd import inputs, ops

pytestmark = pytest.mark.gpu


def _case(M, K, N, step):
    wl = f"noalloc/{M}x{K}x{N}"
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x", step)).cuda()
    g, b = (t.cuda() for t in inputs.layernorm_params(K, wl))
    w = inputs.linear_weight(N, K, wl, "w").cuda()
    dy = inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy", step), std=1e-3).cuda()
    return x, g, b, w, dy


def _backward(noalloc, recipe, x, g, dy, ctx, mf, mb):
    M, K = x.shape
    N = dy.shape[1]
    mb = _clone_meta(mb)
    outs = dict(dx=torch.full((M, K), float("nan"), dtype=torch.bfloat16, device="cuda"),
                dgamma=torch.full((K,), float("nan"), device="cuda"),
                dbeta=torch.full((K,), float("nan"), device="cuda"),
                dw=torch.full((N, K), float("nan"), device="cuda"),
                dbias=torch.full((N,), float("nan"), device="cuda"))
    fn = ops.ln_linear_bwd_noalloc if noalloc else ops.ln_linear_bwd
    fn(recipe, dy, x, g, ctx, mf, mb, outs["dx"], outs["dgamma"], outs["dbeta"], outs["dw"],
       outs["dbias"])
    torch.cuda.synchronize()
    outs["history"], outs["scale"] = mb.history.clone(), mb.scale.clone()
    return outs


def _clone_meta(m):
    c = ops.Meta(m.recipe, m.n_slots, m.kind, init=False)
    c.history.copy_(m.history)
    c.scale.copy_(m.scale)
    c.scale_inv.copy_(m.scale_inv)
    return c


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_noalloc_backward_equals_workspace_backward():
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    for call, (M, K, N) in enumerate([(2048, 768, 2304), (512, 768, 1024)]):
        print(f"no-alloc call {call}: {M} x {K} -> {N}", flush=True)
        x, g, b, w, dy = _case(M, K, N, call)
        mf = ops.Meta(recipe, 2, ops.META_FORWARD)
        mb = ops.Meta(recipe, 1, ops.META_BACKWARD)
        ctx = ops.LinearCtx(M, K, N)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):   # a second step, so the scales are set from a history
            ops.scaling_update(recipe, mf)
            ops.ln_linear_fwd(recipe, x, g, b, w, None, out, mf, ctx)
            ops.scaling_update(recipe, mb)
        ref = _backward(False, recipe, x, g, dy, ctx, mf, mb)
        got = _backward(True, recipe, x, g, dy, ctx, mf, mb)
        for k in ref:
            assert _same_bits(got[k], ref[k]), f"call {call}: {k} differs"
        assert torch.isfinite(ref["dw"]).all() and torch.isfinite(ref["dx"].float()).all()
        assert ref["history"][0, 0] > 0


def test_noalloc_rejects_sizes_beyond_its_array():
    recipe = ops.Recipe()
    M, K, N = 8192, 1024, 4096     # needs more than the 32 MiB array
    assert ops.workspace_size(ops.OP_LN_LINEAR_BWD, M, K, N) > 32 << 20
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    g = torch.empty(K, dtype=torch.bfloat16, device="cuda")
    ctx = ops.LinearCtx(M, K, N)
    mf = ops.Meta(recipe, 2, ops.META_FORWARD)
    mb = ops.Meta(recipe, 1, ops.META_BACKWARD)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((N, K), device="cuda")
    dg = torch.empty(K, device="cuda")
    with pytest.raises(ops.Fp8lnError, match="scratch"):
        ops.ln_linear_bwd_noalloc(recipe, dy, x, g, ctx, mf, mb, dx, dg, dg.clone(), dw)
