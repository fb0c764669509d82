"""GPU parity of the fused modules through the C ABI, step by step against the
oracle's own chain on the same seeded inputs.

Shapes follow the pages' GPT-style workload: hidden 768 with QKV width 2304 and
FFN 3072 at 8 x 32 and 8 x 256 tokens, plus the hidden-2048 / FFN-8192 scale-up
at 64 x 256 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_delayed_scaling_row_amd import inputs, ops
from parity import (assert_gemm_close, assert_vector_close, compare_codes, ln_window, to_np,
                    to_np_bits)

pytestmark = pytest.mark.gpu

OFMT = {ops.FORMAT_E4M3: oracle.FORMAT_E4M3, ops.FORMAT_HYBRID: oracle.FORMAT_HYBRID,
        ops.FORMAT_E5M2: oracle.FORMAT_E5M2}
EPS = float(np.float32(1e-5))
U32 = 2.0 ** -24


def orecipe(r: ops.Recipe):
    return oracle.Recipe(format=OFMT[r.format], amax_history_len=r.amax_history_len,
                         margin=r.margin, ln_eps=r.ln_eps, activation=r.activation)


def f32bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def check_meta(gpu: ops.Meta, om: oracle.Meta, exact_slots, rel_slots, rel=1e-6, what=""):
    gh = gpu.history.cpu().numpy()
    gs = gpu.scale.cpu().numpy()
    for s in exact_slots:
        np.testing.assert_array_equal(f32bits(gh[:, s]), f32bits(om.history[:, s]),
                                      err_msg=f"{what} history slot {s}")
        np.testing.assert_array_equal(f32bits(gs[s]), f32bits(om.scale[s]),
                                      err_msg=f"{what} scale slot {s}")
    for s in rel_slots:
        np.testing.assert_allclose(gh[:, s], om.history[:, s], rtol=rel, atol=0,
                                   err_msg=f"{what} history slot {s}")
        np.testing.assert_allclose(gs[s], om.scale[s], rtol=rel, err_msg=f"{what} scale {s}")


def ln_parts(x_bits, g_bits, b_bits):
    x = oracle.bf16_to_f64(x_bits)
    g = oracle.bf16_to_f64(g_bits)
    y, mean, rstd = oracle.layernorm_fwd(x, g, oracle.bf16_to_f64(b_bits), EPS)
    return (x - mean[:, None]) * rstd[:, None] * g, oracle.bf16_to_f64(b_bits)


def scale_slack(gpu_meta, om, slot, exact):
    """Extra window for a delayed scale that differs from the oracle's by a few
    ulps (its amax history came from an fp32 LayerNorm or GEMM)."""
    gs = float(gpu_meta.scale[slot].item())
    return abs(gs / float(om.scale[slot]) - 1.0) * np.abs(exact)


# ---- LayerNormLinear -----------------------------------------------------------

def run_linear(recipe, M, K, N, steps, workload, backward, check_every=1, reuse_from=None):
    """reuse_from: from this step on the forward reuses the FP8 weight codes of the
    last step that cast the weight (FP8 weight storage), on the GPU and in the
    oracle alike."""
    dev = "cuda"
    g, b = inputs.layernorm_params(K, workload)
    w = inputs.linear_weight(N, K, workload, "weight")
    bias = inputs.normal_bf16((N,), inputs.seed_for(workload, "bias"), std=0.1)
    gd, bd, wd, biasd = g.to(dev), b.to(dev), w.to(dev), bias.to(dev)
    mf, mb = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=backward)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dgamma = torch.empty(K, dtype=torch.float32, device=dev)
    dbeta = torch.empty(K, dtype=torch.float32, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    dbias = torch.empty(N, dtype=torch.float32, device=dev)
    orc = orecipe(recipe)
    omf, omb = oracle.linear_fwd_meta(orc), oracle.linear_bwd_meta(orc)
    ffmt, bfmt = oracle.fwd_format(orc), oracle.bwd_format(orc)
    gbits, bbits, wbits, biasbits = map(to_np_bits, (g, b, w, bias))
    cached = None
    for step in range(steps):
        reuse = reuse_from is not None and step >= reuse_from
        ctx.reuse_weight_codes = reuse
        x = inputs.normal_bf16((M, K), inputs.seed_for(workload, "x", step))
        xd = x.to(dev)
        ops.scaling_update(recipe, mf)
        ops.ln_linear_fwd(recipe, xd, gd, bd, wd, biasd, out, mf, ctx)
        oracle.scaling_update(omf, orc.margin)
        xbits = to_np_bits(x)
        oout, octx = oracle.ln_linear_fwd(orc, omf, xbits, gbits, bbits, wbits, biasbits,
                                          cached_w=cached if reuse else None)
        if not reuse:
            cached = (octx["w_q"], octx["w_sinv"])
        if backward:
            dy = inputs.normal_bf16((M, N), inputs.seed_for(workload, "dy", step), std=1e-3)
            ops.scaling_update(recipe, mb)
            ops.ln_linear_bwd(recipe, dy.to(dev), xd, gd, ctx, mf, mb, dx, dgamma, dbeta, dw,
                              dbias)
            oracle.scaling_update(omb, orc.margin)
            og = oracle.ln_linear_bwd(orc, omf, omb, to_np_bits(dy), octx, xbits, gbits)
        torch.cuda.synchronize()
        if step % check_every and step != steps - 1:
            continue
        tag = f"step {step}"
        assert_gemm_close(to_np(out), oout, what=f"{tag} out")
        gx, beta = ln_parts(xbits, gbits, bbits)
        s0 = float(omf.scale[0])
        exact = octx["y"] * s0
        compare_codes(ctx.ln_q.cpu().numpy(), exact, ffmt,
                      ln_window(gx, beta, s0, exact) + scale_slack(mf, omf, 0, exact))
        if reuse:
            np.testing.assert_array_equal(ctx.w_q.cpu().numpy(), octx["w_q"])
        else:
            wex = oracle.bf16_to_f64(wbits) * float(omf.scale[1])
            compare_codes(ctx.w_q.cpu().numpy(), wex, ffmt, 0.0)
        assert ctx.w_scale_inv.item() == float(octx["w_sinv"])
        if backward:
            assert torch.equal(ctx.ln_qt, ctx.ln_q.t().contiguous())
            assert torch.equal(ctx.w_qt, ctx.w_q.t().contiguous())
        check_meta(mf, omf, exact_slots=[1], rel_slots=[0], what=f"{tag} fwd")
        if backward:
            check_meta(mb, omb, exact_slots=[0], rel_slots=[], what=f"{tag} bwd")
            assert_gemm_close(to_np(dx), og["dx"], alarm=1e-2, what=f"{tag} dx")
            assert_gemm_close(dw.cpu().numpy(), og["dw"], alarm=5e-3, what=f"{tag} dW")
            assert_vector_close(dgamma.cpu().numpy(), og["dgamma"], 2e-3, f"{tag} dgamma")
            assert_vector_close(dbeta.cpu().numpy(), og["dbeta"], 2e-3, f"{tag} dbeta")
            assert_vector_close(dbias.cpu().numpy(), og["dbias"], 1e-5, f"{tag} dbias")


def test_ln_linear_fwd_module_tour_16_steps():
    """LayerNormLinear(768, 2304) on 8 x 32 tokens, HYBRID, history 16, 16 steps
    with fresh inputs so the history fills."""
    run_linear(ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16), 256, 768, 2304, 16,
               "c0", backward=False)


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3, ops.FORMAT_E5M2])
def test_ln_linear_fwd_bwd_2048_tokens(fmt):
    run_linear(ops.Recipe(format=fmt, amax_history_len=16), 2048, 768, 2304, 3, f"c3/{fmt}",
               backward=True)


@pytest.mark.parametrize("M,K,N", [(48, 64, 80), (16, 16, 16), (144, 256, 400)])
def test_ln_linear_small_and_ragged(M, K, N):
    run_linear(ops.Recipe(amax_history_len=4, margin=1), M, K, N, 5, f"lin/{M}/{K}/{N}",
               backward=True)


def test_ln_linear_fp8_weight_storage():
    """Steps 2.. reuse the weight codes cast at step 1: the forward skips the
    weight cast, the GEMMs use the stored scale_inv, the weight slot records no
    amax (its history rows stay zero, as in the oracle), and every output still
    matches the oracle run in the same mode."""
    run_linear(ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=4), 256, 768, 2304, 6,
               "lin/fp8-weights", backward=True, reuse_from=2)


def test_ln_linear_fwd_ragged_tokens_forward_only():
    run_linear(ops.Recipe(), 37, 768, 2304, 2, "lin-ragged", backward=False)


# ---- Linear (no LayerNorm) -------------------------------------------------------

def run_plain_linear(recipe, M, K, N, steps, workload, backward, reuse_from=None,
                     with_bias=True):
    """Linear's chain step by step against the oracle.  Every FP8 code here comes
    from a bf16 value times a binary32 scale, so codes, amaxes and scales are
    compared bit for bit; the GEMM outputs follow the GEMM rule."""
    dev = "cuda"
    w = inputs.linear_weight(N, K, workload, "weight")
    bias = inputs.normal_bf16((N,), inputs.seed_for(workload, "bias"), std=0.1)
    wd = w.to(dev)
    biasd = bias.to(dev) if with_bias else None
    mf, mb = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=backward)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    dbias = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
    orc = orecipe(recipe)
    omf, omb = oracle.linear_fwd_meta(orc), oracle.linear_bwd_meta(orc)
    ffmt, bfmt = oracle.fwd_format(orc), oracle.bwd_format(orc)
    wbits = to_np_bits(w)
    biasbits = to_np_bits(bias) if with_bias else None
    cached = None
    for step in range(steps):
        reuse = reuse_from is not None and step >= reuse_from
        ctx.reuse_weight_codes = reuse
        x = inputs.normal_bf16((M, K), inputs.seed_for(workload, "x", step))
        ops.scaling_update(recipe, mf)
        ops.linear_fwd(recipe, x.to(dev), wd, biasd, out, mf, ctx)
        oracle.scaling_update(omf, orc.margin)
        oout, octx = oracle.linear_fwd(orc, omf, to_np_bits(x), wbits, biasbits,
                                       cached_w=cached if reuse else None)
        if not reuse:
            cached = (octx["w_q"], octx["w_sinv"])
        if backward:
            dy = inputs.normal_bf16((M, N), inputs.seed_for(workload, "dy", step), std=1e-3)
            ops.scaling_update(recipe, mb)
            ops.linear_bwd(recipe, dy.to(dev), ctx, mf, mb, dx, dw, dbias)
            oracle.scaling_update(omb, orc.margin)
            og = oracle.linear_bwd(orc, omf, omb, to_np_bits(dy), octx)
        torch.cuda.synchronize()
        tag = f"step {step}"
        np.testing.assert_array_equal(ctx.ln_q.cpu().numpy(), octx["x_q"], err_msg=f"{tag} x_q")
        np.testing.assert_array_equal(ctx.w_q.cpu().numpy(), octx["w_q"], err_msg=f"{tag} w_q")
        assert ctx.w_scale_inv.item() == float(octx["w_sinv"])
        check_meta(mf, omf, exact_slots=[0, 1], rel_slots=[], what=f"{tag} fwd")
        if M > 0:
            assert_gemm_close(to_np(out), oout, alarm=5e-3, what=f"{tag} out")
        if backward:
            assert torch.equal(ctx.ln_qt, ctx.ln_q.t().contiguous())
            assert torch.equal(ctx.w_qt, ctx.w_q.t().contiguous())
            check_meta(mb, omb, exact_slots=[0], rel_slots=[], what=f"{tag} bwd")
            if M > 0:
                assert_gemm_close(to_np(dx), og["dx"], alarm=5e-3, what=f"{tag} dx")
                assert_gemm_close(dw.cpu().numpy(), og["dw"], alarm=1e-3, what=f"{tag} dW")
                assert_vector_close(dbias.cpu().numpy(), og["dbias"], 1e-5, f"{tag} dbias")
            else:
                assert not dw.any().item(), "dW of zero tokens must be zero"
                assert not dbias.any().item(), "dbias of zero tokens must be zero"


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3, ops.FORMAT_E5M2])
def test_linear_fwd_bwd_2048_tokens(fmt):
    """Linear(768, 2304) on 8 x 256 tokens, three steps."""
    run_plain_linear(ops.Recipe(format=fmt, amax_history_len=16), 2048, 768, 2304, 3,
                     f"plin/{fmt}", backward=True)


@pytest.mark.parametrize("M,K,N", [(48, 64, 80), (16, 16, 16), (144, 256, 400), (0, 64, 32)])
def test_linear_small_ragged_and_empty(M, K, N):
    run_plain_linear(ops.Recipe(amax_history_len=4, margin=1), M, K, N, 3,
                     f"plin/{M}/{K}/{N}", backward=True, with_bias=(M != 16))


def test_linear_forward_only_ragged_tokens():
    run_plain_linear(ops.Recipe(), 37, 768, 2304, 2, "plin-ragged", backward=False)


def test_linear_fp8_weight_storage():
    run_plain_linear(ops.Recipe(amax_history_len=4), 256, 768, 2304, 5, "plin/fp8-weights",
                     backward=True, reuse_from=2)


def test_linear_large_tiles():
    """A shape that takes the large GEMM tiles in all three products (long K in
    the weight gradient)."""
    run_plain_linear(ops.Recipe(amax_history_len=2), 4096, 2048, 2048, 1, "plin/large",
                     backward=True)


# ---- LayerNormMLP --------------------------------------------------------------

MFMA_DOT_REL = 2.0 ** -10


def gelu_code_window(ln_q, w1_q, fmt, alpha, h, scale, K, act=ops.GELU_TANH):
    """GEMM-fed window for the GELU output's codes.  The FP8 MFMA's 128-term dot
    products carry about 13-14 bits relative to their sum of |a b| (measured
    worst case 3.2e-4 on full-range random codes); the fp32 accumulator adds are
    exact to 2^-24.  Bound: 2^-10 * alpha * sum_k |a b| for h, then through
    GELU', plus the epilogue's roundings and the fp32 GELU."""
    a = oracle.fp8_decode(ln_q & 0x7F, fmt)
    b = oracle.fp8_decode(w1_q & 0x7F, fmt)
    abs_sum = a @ b.T
    dh = MFMA_DOT_REL * float(alpha) * abs_sum + 4 * U32 * np.abs(h)
    gelu, gelu_grad = ((oracle.gelu_erf, oracle.gelu_erf_grad) if act == ops.GELU_ERF
                       else (oracle.gelu_tanh, oracle.gelu_tanh_grad))
    dg = np.abs(gelu_grad(h)) * dh + 1e-6 * np.abs(gelu(h)) + 2e-7 * np.abs(h)
    return float(scale) * dg


def run_mlp(recipe, M, H, F, steps, workload, backward, sample_rows=None, reuse_from=None):
    dev = "cuda"
    g, b = inputs.layernorm_params(H, workload)
    w1 = inputs.linear_weight(F, H, workload, "w1")
    w2 = inputs.linear_weight(H, F, workload, "w2")
    b1 = inputs.normal_bf16((F,), inputs.seed_for(workload, "b1"), std=0.1)
    b2 = inputs.normal_bf16((H,), inputs.seed_for(workload, "b2"), std=0.1)
    gd, bd, w1d, w2d, b1d, b2d = (t.to(dev) for t in (g, b, w1, w2, b1, b2))
    mf, mb = ops.mlp_metas(recipe)
    ctx = ops.MlpCtx(M, H, F, training=True)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    dgamma = torch.empty(H, dtype=torch.float32, device=dev)
    dbeta = torch.empty(H, dtype=torch.float32, device=dev)
    dw1 = torch.empty((F, H), dtype=torch.float32, device=dev)
    dw2 = torch.empty((H, F), dtype=torch.float32, device=dev)
    db1 = torch.empty(F, dtype=torch.float32, device=dev)
    db2 = torch.empty(H, dtype=torch.float32, device=dev)
    orc = orecipe(recipe)
    omf, omb = oracle.mlp_fwd_meta(orc), oracle.mlp_bwd_meta(orc)
    ffmt = oracle.fwd_format(orc)
    gbits, bbits, w1bits, w2bits, b1bits, b2bits = map(to_np_bits, (g, b, w1, w2, b1, b2))
    rows = slice(None) if sample_rows is None else sample_rows
    cached = None
    for step in range(steps):
        reuse = reuse_from is not None and step >= reuse_from
        ctx.reuse_weight_codes = reuse
        x = inputs.normal_bf16((M, H), inputs.seed_for(workload, "x", step), device=dev)
        ops.scaling_update(recipe, mf)
        ops.ln_mlp_fwd(recipe, x, gd, bd, w1d, b1d, w2d, b2d, out, mf, ctx)
        xbits = to_np_bits(x)
        oracle.scaling_update(omf, orc.margin)
        oout, octx = oracle.ln_mlp_fwd(orc, omf, xbits, gbits, bbits, w1bits, b1bits, w2bits,
                                       b2bits, cached_w=cached if reuse else None)
        if not reuse:
            cached = ((octx["w1_q"], octx["w1_sinv"]), (octx["w2_q"], octx["w2_sinv"]))
        if backward:
            dy = inputs.normal_bf16((M, H), inputs.seed_for(workload, "dy", step), std=1e-3,
                                    device=dev)
            ops.scaling_update(recipe, mb)
            ops.ln_mlp_bwd(recipe, dy, x, gd, ctx, mf, mb, dx, dgamma, dbeta, dw1, db1, dw2, db2)
            oracle.scaling_update(omb, orc.margin)
            og = oracle.ln_mlp_bwd(orc, omf, omb, to_np_bits(dy), octx, xbits, gbits)
        torch.cuda.synchronize()
        tag = f"step {step}"
        # one LayerNorm code that the rule lets differ moves a whole fc1 row by ~1 %
        # and its GELU codes by several steps, so the row alarm is 5e-2 here
        assert_gemm_close(to_np(out)[rows], oout[rows], alarm=5e-2, what=f"{tag} out")
        assert_gemm_close(to_np(ctx.h)[rows], octx["h"][rows], alarm=5e-2, what=f"{tag} h")
        gx, beta = ln_parts(xbits[rows], gbits, bbits)
        s0 = float(omf.scale[0])
        exact = octx["y"][rows] * s0
        compare_codes(ctx.ln_q.cpu().numpy()[rows], exact, ffmt,
                      ln_window(gx, beta, s0, exact) + scale_slack(mf, omf, 0, exact))
        alpha = np.float32(omf.scale_inv[0]) * np.float32(octx["w1_sinv"])
        np.testing.assert_array_equal(ctx.w_scale_inv.cpu().numpy(),
                                      np.array([octx["w1_sinv"], octx["w2_sinv"]], np.float32))
        if reuse:
            np.testing.assert_array_equal(ctx.w1_q.cpu().numpy(), octx["w1_q"])
            np.testing.assert_array_equal(ctx.w2_q.cpu().numpy(), octx["w2_q"])
        s2 = float(omf.scale[2])
        gq = ctx.g_q.cpu().numpy()[rows]
        win = gelu_code_window(octx["ln_q"][rows], octx["w1_q"], ffmt, alpha, octx["h"][rows],
                               s2, H, recipe.activation)
        # LayerNorm codes the rule let differ (one step next to a midpoint) move the
        # whole fc1 row: add their effect through |W1| and the largest GELU' (1.13)
        d_ln = np.abs(oracle.fp8_decode(ctx.ln_q.cpu().numpy()[rows], ffmt) -
                      oracle.fp8_decode(octx["ln_q"][rows], ffmt))
        if d_ln.any():
            w1abs = np.abs(oracle.fp8_decode(octx["w1_q"], ffmt))
            win = win + s2 * 1.13 * float(alpha) * (d_ln @ w1abs.T)
        stats = compare_codes(gq, octx["g"][rows] * s2, ffmt,
                              win + scale_slack(mf, omf, 2, octx["g"][rows] * s2))
        assert torch.equal(ctx.g_qt, ctx.g_q.t().contiguous())
        check_meta(mf, omf, exact_slots=[1, 3], rel_slots=[0], what=f"{tag} fwd")
        np.testing.assert_allclose(mf.history.cpu().numpy()[:, 2], omf.history[:, 2], rtol=1e-4)
        if backward:
            check_meta(mb, omb, exact_slots=[0], rel_slots=[1], rel=5e-3, what=f"{tag} bwd")
            # dH is a GEMM output cast to E5M2 (25 % steps): a code the rule lets
            # differ moves a row of dLN / dW1 by about a percent
            assert_gemm_close(to_np(dx)[rows], og["dx"][rows], alarm=5e-2, what=f"{tag} dx")
            assert_gemm_close(dw1.cpu().numpy(), og["dw1"], alarm=5e-2, what=f"{tag} dW1")
            assert_gemm_close(dw2.cpu().numpy(), og["dw2"], alarm=5e-3, what=f"{tag} dW2")
            assert_vector_close(db1.cpu().numpy(), og["db1"], 1e-3, f"{tag} db1")
            assert_vector_close(db2.cpu().numpy(), og["db2"], 1e-5, f"{tag} db2")
            assert_vector_close(dgamma.cpu().numpy(), og["dgamma"], 5e-3, f"{tag} dgamma")
            assert_vector_close(dbeta.cpu().numpy(), og["dbeta"], 5e-3, f"{tag} dbeta")
        print(f"{workload} {tag}: g codes {stats}")


def test_ln_mlp_fwd_2048_tokens():
    """LayerNormMLP 768 -> 3072 -> 768 on 8 x 256 tokens, E4M3 on both GEMM
    inputs with separate histories, history 16."""
    run_mlp(ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=16), 2048, 768, 3072, 4,
            "c2", backward=False)


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3, ops.FORMAT_E5M2])
def test_ln_mlp_fwd_bwd_small(fmt):
    run_mlp(ops.Recipe(format=fmt, amax_history_len=8), 256, 256, 1024, 3, f"mlp/{fmt}",
            backward=True)


def test_ln_mlp_ragged_tiles():
    run_mlp(ops.Recipe(), 48, 80, 144, 3, "mlp-ragged", backward=True)


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3])
def test_ln_mlp_erf_gelu(fmt):
    """LayerNormMLP with the erf form of GELU (nn.GELU() of the mirror block)."""
    run_mlp(ops.Recipe(format=fmt, amax_history_len=8, activation=ops.GELU_ERF), 256, 256,
            1024, 3, f"mlp-erf/{fmt}", backward=True)


def test_ln_mlp_fp8_weight_storage():
    """Both weights' codes cast at step 1 are reused from step 2 on (forward and
    backward), matching the oracle run in the same mode."""
    run_mlp(ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=4), 256, 256, 1024, 5,
            "mlp/fp8-weights", backward=True, reuse_from=2)


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3])
def test_ln_mlp_full_layer_sampled(fmt):
    """One scale-up layer (16384 tokens, 2048 -> 8192 -> 2048), history 1024,
    two steps; row-wise results compared on 64 sampled tokens, everything that
    reduces over tokens (amaxes, weight gradients, bias gradients) in full."""
    rows = np.unique(np.concatenate([[0, 16383],
                                     np.random.default_rng(2).integers(0, 16384, 62)]))
    run_mlp(ops.Recipe(format=fmt, amax_history_len=1024), 16384, 2048, 8192, 2, f"c4/{fmt}",
            backward=True, sample_rows=rows)


def test_modules_are_deterministic():
    r = ops.Recipe()
    M, H, F = 512, 768, 3072
    x = inputs.normal_bf16((M, H), 1, device="cuda")
    g, b = inputs.layernorm_params(H, "det", device="cuda")
    w1 = inputs.linear_weight(F, H, "det", "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, "det", "w2", device="cuda")
    dy = inputs.normal_bf16((M, H), 2, std=1e-3, device="cuda")
    results = []
    for _ in range(2):
        mf, mb = ops.mlp_metas(r)
        ctx = ops.MlpCtx(M, H, F)
        out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty_like(out)
        grads = [torch.empty(H, device="cuda"), torch.empty(H, device="cuda"),
                 torch.empty((F, H), device="cuda"), torch.empty(F, device="cuda"),
                 torch.empty((H, F), device="cuda"), torch.empty(H, device="cuda")]
        for _step in range(2):
            ops.scaling_update(r, mf)
            ops.ln_mlp_fwd(r, x, g, b, w1, None, w2, None, out, mf, ctx)
            ops.scaling_update(r, mb)
            ops.ln_mlp_bwd(r, dy, x, g, ctx, mf, mb, dx, *grads)
        torch.cuda.synchronize()
        results.append([out.clone(), dx.clone(), mf.history.clone(), mb.history.clone()] +
                       [t.clone() for t in grads])
    for a, c in zip(*results):
        assert torch.equal(a, c)


def _oracle_meta(gpu: ops.Meta, fmt, n):
    """The GPU state block as an oracle Meta (identical-input mode)."""
    return oracle.Meta(gpu.history.cpu().numpy().copy(), gpu.scale.cpu().numpy().copy(),
                       gpu.scale_inv.cpu().numpy().copy(), [fmt] * n)


def _sampled_weight_grads(orc, om_f, om_b, x_bits, dy_bits, g_bits, b_bits, w1_bits, w2_bits, fs):
    """The oracle's token-reduced backward results of one LayerNormMLP layer
    (no biases) over every token, at the fc1 output features fs: rows fs of dW1,
    columns fs of dW2, db1[fs] and all of db2.  The oracle's own steps (LayerNorm
    + cast, weight casts, FP8 GEMMs, GELU, gradient casts) run on the whole token
    set; only the fc1 columns fs of each product are formed, which is all these
    results depend on.  The state blocks are not modified."""
    ffmt, bfmt = oracle.fwd_format(orc), oracle.bwd_format(orc)
    gelu, gelu_grad = ((oracle.gelu_erf, oracle.gelu_erf_grad) if orc.activation == ops.GELU_ERF
                       else (oracle.gelu_tanh, oracle.gelu_tanh_grad))
    ln = oracle.ln_cast_amax(x_bits, g_bits, b_bits, orc.eps64, om_f.scale[0], ffmt)
    w1_q, _ = oracle.cast_amax(oracle.bf16_to_f64(w1_bits), om_f.scale[1], ffmt)
    w2_q, _ = oracle.cast_amax(oracle.bf16_to_f64(w2_bits), om_f.scale[3], ffmt)
    h = oracle.fp8_gemm_tn(ln["q"], ffmt, w1_q[fs], ffmt, om_f.scale_inv[0], om_f.scale_inv[1])
    g_q, _ = oracle.cast_amax(gelu(h), om_f.scale[2], ffmt)
    dy = oracle.bf16_to_f64(dy_bits)
    dy_q, _ = oracle.cast_amax(dy, om_b.scale[0], bfmt)
    dg = oracle.fp8_gemm_tn(dy_q, bfmt, np.ascontiguousarray(w2_q.T[fs]), ffmt,
                            om_b.scale_inv[0], om_f.scale_inv[3])
    dh = dg * gelu_grad(oracle.bf16_to_f64(oracle.f64_to_bf16_bits(h)))
    dh_q, _ = oracle.cast_amax(dh, om_b.scale[1], bfmt)
    return dict(
        dw1_rows=oracle.fp8_gemm_tn(dh_q.T, bfmt, ln["q"].T, ffmt, om_b.scale_inv[1],
                                    om_f.scale_inv[0]),
        dw2_cols=oracle.fp8_gemm_tn(dy_q.T, bfmt, g_q.T, ffmt, om_b.scale_inv[0],
                                    om_f.scale_inv[2]),
        db1=dh.sum(axis=0), db2=dy.sum(axis=0))


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3])
def test_ln_mlp_x12_chain_layers_0_5_11(fmt):
    """The 12-layer scale-up chain (16384 tokens, 2048 -> 8192 -> 2048, history
    1024, each layer's output the next one's input, as the benchmark runs it), two
    steps.  At layers 0, 5 and 11 of the second step the oracle takes the GPU's own
    layer input, incoming gradient and state blocks (identical-input mode, so FP8
    rounding flips do not compound across layers) and the layer's row-wise results
    are compared on sampled tokens."""
    M, H, F, L = 16384, 2048, 8192, 12
    recipe = ops.Recipe(format=fmt, amax_history_len=1024)
    orc = orecipe(recipe)
    ffmt, bfmt = oracle.fwd_format(orc), oracle.bwd_format(orc)
    wl = f"ln_mlp_x{L}_{M}x{H}x{F}"
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(12).integers(0, M, 30)]))
    rows_t = torch.from_numpy(rows).cuda()
    x0 = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"), device="cuda")
    dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-3, device="cuda")
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    layers = []
    for l in range(L):
        g, b = inputs.layernorm_params(H, f"{wl}/{l}")
        w1 = inputs.linear_weight(F, H, f"{wl}/{l}", "w1")
        w2 = inputs.linear_weight(H, F, f"{wl}/{l}", "w2")
        mf, mb = ops.mlp_metas(recipe)
        layers.append(dict(bits=[to_np_bits(t) for t in (g, b, w1, w2)],
                           dev=[t.cuda() for t in (g, b, w1, w2)], mf=mf, mb=mb,
                           ctx=ops.MlpCtx(M, H, F),
                           out=torch.empty((M, H), dtype=torch.bfloat16, device="cuda"),
                           grads=[f32(H), f32(H), f32(F, H), f32(F), f32(H, F), f32(H)]))
    dxs = [torch.empty((M, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    checks = (0, 5, 11)
    saved = {}
    for step in range(2):
        x = x0
        for l, d in enumerate(layers):
            g, b, w1, w2 = d["dev"]
            ops.scaling_update(recipe, d["mf"])
            if step == 1 and l in checks:
                saved[l] = dict(x=to_np_bits(x[rows_t]), mf=_oracle_meta(d["mf"], ffmt, 4),
                                x_full=to_np_bits(x))
            ops.ln_mlp_fwd(recipe, x, g, b, w1, None, w2, None, d["out"], d["mf"], d["ctx"])
            x = d["out"]
        grad = dy
        for i in range(L):
            l = L - 1 - i
            d = layers[l]
            xin = x0 if l == 0 else layers[l - 1]["out"]
            ops.scaling_update(recipe, d["mb"])
            if step == 1 and l in checks:
                saved[l]["dy"] = to_np_bits(grad[rows_t])
                saved[l]["dy_full"] = to_np_bits(grad)
                saved[l]["mb"] = _oracle_meta(d["mb"], bfmt, 2)
            dx = dxs[i % 2]
            ops.ln_mlp_bwd(recipe, grad, xin, d["dev"][0], d["ctx"], d["mf"], d["mb"], dx,
                           *d["grads"])
            if step == 1 and l in checks:
                saved[l]["dx"] = to_np(dx[rows_t])
            grad = dx
    torch.cuda.synchronize()
    for l in checks:
        d, sv = layers[l], saved[l]
        gbits, bbits, w1bits, w2bits = d["bits"]
        omf, omb = sv["mf"], sv["mb"]
        oout, octx = oracle.ln_mlp_fwd(orc, omf, sv["x"], gbits, bbits, w1bits, None, w2bits,
                                       None)
        og = oracle.ln_mlp_bwd(orc, omf, omb, sv["dy"], octx, sv["x"], gbits)
        ctx = d["ctx"]
        tag = f"layer {l}"
        assert_gemm_close(to_np(d["out"][rows_t]), oout, alarm=5e-2, what=f"{tag} out")
        assert_gemm_close(to_np(ctx.h[rows_t]), octx["h"], alarm=5e-2, what=f"{tag} h")
        gx, beta = ln_parts(sv["x"], gbits, bbits)
        s0 = float(omf.scale[0])
        exact = octx["y"] * s0
        lnq = ctx.ln_q[rows_t].cpu().numpy()
        compare_codes(lnq, exact, ffmt, ln_window(gx, beta, s0, exact))
        np.testing.assert_array_equal(
            ctx.w1_q.cpu().numpy(), octx["w1_q"], err_msg=f"{tag} fc1 weight codes")
        alpha = np.float32(omf.scale_inv[0]) * np.float32(octx["w1_sinv"])
        s2 = float(omf.scale[2])
        win = gelu_code_window(octx["ln_q"], octx["w1_q"], ffmt, alpha, octx["h"], s2, H,
                               recipe.activation)
        d_ln = np.abs(oracle.fp8_decode(lnq, ffmt) - oracle.fp8_decode(octx["ln_q"], ffmt))
        if d_ln.any():
            w1abs = np.abs(oracle.fp8_decode(octx["w1_q"], ffmt))
            win = win + s2 * 1.13 * float(alpha) * (d_ln @ w1abs.T)
        stats = compare_codes(ctx.g_q[rows_t].cpu().numpy(), octx["g"] * s2, ffmt, win)
        assert_gemm_close(sv["dx"], og["dx"], alarm=5e-2, what=f"{tag} dx")
        # the token-reduced results over all 16384 tokens, at sampled fc1 features
        fs = np.unique(np.concatenate([[0, F - 1], np.random.default_rng(l).integers(0, F, 6)]))
        ref = _sampled_weight_grads(orc, sv["mf"], sv["mb"], sv["x_full"], sv["dy_full"],
                                    gbits, bbits, w1bits, w2bits, fs)
        gdw1, gdb1, gdw2, gdb2 = (t.cpu().numpy() for t in
                                  (d["grads"][2], d["grads"][3], d["grads"][4], d["grads"][5]))
        assert_gemm_close(gdw1[fs], ref["dw1_rows"], alarm=5e-2, what=f"{tag} dW1 rows")
        assert_gemm_close(gdw2[:, fs].T, ref["dw2_cols"].T, alarm=5e-2,
                          what=f"{tag} dW2 columns")
        assert_vector_close(gdb1[fs], ref["db1"], 1e-3, f"{tag} db1")
        assert_vector_close(gdb2, ref["db2"], 1e-5, f"{tag} db2")
        print(f"{fmt} {tag}: g codes {stats}")


# ---- the fused forward front equals the standalone kernels -----------------------

def _set_meta(meta, scales):
    meta.scale.copy_(torch.tensor(scales, dtype=torch.float32))
    meta.scale_inv.copy_(1.0 / meta.scale)
    meta.history.zero_()


@pytest.mark.parametrize("M,K,N,fmt", [(256, 768, 2304, ops.FORMAT_HYBRID),
                                       (80, 1008, 208, ops.FORMAT_E5M2),
                                       (2048, 768, 2304, ops.FORMAT_E4M3)],
                         ids=["8x32_tokens", "ragged", "2048_tokens"])
def test_ln_linear_fwd_equals_standalone_entry_points(M, K, N, fmt):
    """At small shapes the forward runs the LayerNorm rows and the weight cast in
    one launch; its codes, row statistics, amaxes and output must equal, bit for
    bit, those of the standalone LayerNorm+cast, cast and GEMM entry points fed
    the same scales."""
    recipe = ops.Recipe(format=fmt, amax_history_len=16)
    wl = f"prologue/{M}x{K}x{N}"
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x"), std=2.0, mean=0.5).cuda()
    g, b = (t.cuda() for t in inputs.layernorm_params(K, wl))
    w = inputs.linear_weight(N, K, wl, "w").cuda()
    bias = inputs.normal_bf16((N,), inputs.seed_for(wl, "bias"), std=0.1).cuda()
    ma, _ = ops.linear_metas(recipe)
    mb, _ = ops.linear_metas(recipe)
    for m in (ma, mb):
        _set_meta(m, [3.25, 1791.0])
    ctx = ops.LinearCtx(M, K, N, training=True)
    out_a = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.ln_linear_fwd(recipe, x, g, b, w, bias, out_a, ma, ctx)

    f = ops.fwd_fp8(recipe)
    ln_q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    ln_qt = torch.empty((K, M), dtype=torch.uint8, device="cuda")
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    w_q = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    w_qt = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    out_b = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.ln_cast_amax(recipe, x, g, b, f, mb.scale[0:1], mb.amax_ptr(0), ln_q, ln_qt, mean, rstd)
    ops.cast_amax(w, f, mb.scale[1:2], mb.amax_ptr(1), w_q, w_qt)
    ops.gemm(ln_q, f, w_q, f, mb.scale_inv[0:1], mb.scale_inv[1:2], out_b, bias)
    torch.cuda.synchronize()
    assert torch.equal(ctx.ln_q, ln_q) and torch.equal(ctx.ln_qt, ln_qt)
    assert torch.equal(ctx.w_q, w_q) and torch.equal(ctx.w_qt, w_qt)
    assert torch.equal(ctx.mean.view(torch.int32), mean.view(torch.int32))
    assert torch.equal(ctx.rstd.view(torch.int32), rstd.view(torch.int32))
    assert torch.equal(ma.history.view(torch.int32), mb.history.view(torch.int32))
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert float(ctx.w_scale_inv.item()) == float(mb.scale_inv[1].item())


@pytest.mark.parametrize("M,H,F", [(2048, 768, 3072), (96, 512, 1040)])
def test_ln_mlp_fwd_front_equals_standalone_entry_points(M, H, F):
    """The MLP forward's fused front (LayerNorm rows and both weight casts in one
    launch) against the standalone entry points, bit for bit: LayerNorm codes,
    statistics, weight codes and the amaxes of those three slots."""
    recipe = ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=16)
    wl = f"prologue-mlp/{M}x{H}x{F}"
    x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x")).cuda()
    g, b = (t.cuda() for t in inputs.layernorm_params(H, wl))
    w1 = inputs.linear_weight(F, H, wl, "w1").cuda()
    w2 = inputs.linear_weight(H, F, wl, "w2").cuda()
    ma, _ = ops.mlp_metas(recipe)
    mb, _ = ops.mlp_metas(recipe)
    for m in (ma, mb):
        _set_meta(m, [5.5, 2100.0, 11.0, 1900.0])
    ctx = ops.MlpCtx(M, H, F, training=True)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ops.ln_mlp_fwd(recipe, x, g, b, w1, None, w2, None, out, ma, ctx)
    f = ops.fwd_fp8(recipe)
    ln_q = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    w1_q, w1_qt = (torch.empty(s, dtype=torch.uint8, device="cuda") for s in ((F, H), (H, F)))
    w2_q, w2_qt = (torch.empty(s, dtype=torch.uint8, device="cuda") for s in ((H, F), (F, H)))
    ops.ln_cast_amax(recipe, x, g, b, f, mb.scale[0:1], mb.amax_ptr(0), ln_q, None, mean, rstd)
    ops.cast_amax(w1, f, mb.scale[1:2], mb.amax_ptr(1), w1_q, w1_qt)
    ops.cast_amax(w2, f, mb.scale[3:4], mb.amax_ptr(3), w2_q, w2_qt)
    torch.cuda.synchronize()
    assert torch.equal(ctx.ln_q, ln_q)
    assert torch.equal(ctx.mean.view(torch.int32), mean.view(torch.int32))
    assert torch.equal(ctx.rstd.view(torch.int32), rstd.view(torch.int32))
    assert torch.equal(ctx.w1_q, w1_q) and torch.equal(ctx.w1_qt, w1_qt)
    assert torch.equal(ctx.w2_q, w2_q) and torch.equal(ctx.w2_qt, w2_qt)
    for s in (0, 1, 3):
        assert ma.history[0, s].view(torch.int32).item() == mb.history[0, s].view(torch.int32).item()


# ---- the pages' workloads over their full step counts ---------------------------

def test_ln_mlp_fwd_2048_tokens_16_steps():
    """LayerNormMLP 768 -> 3072 -> 768 on 8 x 256 tokens, E4M3 on both GEMM inputs
    with separate histories of length 16, over 16 steps (the history fills), each
    step against the oracle's own chain."""
    run_mlp(ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=16), 2048, 768, 3072, 16,
            "c2-16", backward=False)


# ---- checkpoint and resume of the FP8 state ---------------------------------------

def _mlp_run(recipe, M, H, F, steps, first, state, wl):
    """Steps first .. steps-1 of a LayerNormMLP training loop starting from
    `state` (state_dicts of both metas, or None for fresh ones); returns the
    outputs of every step and the final state."""
    g, b = inputs.layernorm_params(H, wl, device="cuda")
    w1 = inputs.linear_weight(F, H, wl, "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, wl, "w2", device="cuda")
    mf, mb = ops.mlp_metas(recipe)
    if state is not None:
        mf.load_state_dict(state[0])
        mb.load_state_dict(state[1])
    ctx = ops.MlpCtx(M, H, F)
    results = []
    for step in range(first, steps):
        x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x", step), device="cuda")
        dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy", step), std=1e-3, device="cuda")
        out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty_like(out)
        grads = [torch.empty(H, device="cuda"), torch.empty(H, device="cuda"),
                 torch.empty((F, H), device="cuda"), torch.empty(F, device="cuda"),
                 torch.empty((H, F), device="cuda"), torch.empty(H, device="cuda")]
        ops.scaling_update(recipe, mf)
        ops.ln_mlp_fwd(recipe, x, g, b, w1, None, w2, None, out, mf, ctx)
        ops.scaling_update(recipe, mb)
        ops.ln_mlp_bwd(recipe, dy, x, g, ctx, mf, mb, dx, *grads)
        results.append([out, dx, ctx.g_q.clone(), mf.history.clone(), mb.history.clone(),
                        mf.scale.clone(), mb.scale.clone()] + grads)
    torch.cuda.synchronize()
    return results, (mf.state_dict(), mb.state_dict())


@pytest.mark.parametrize("fmt", [ops.FORMAT_HYBRID, ops.FORMAT_E4M3])
def test_resume_from_a_checkpoint_is_bit_identical(fmt):
    """The FP8 state (scale, scale_inv, amax history per module and direction,
    as the tutorial's fp8_meta holds it) is everything a step carries over:
    restoring a snapshot taken after step k into fresh state blocks and running
    steps k+1 .. n gives, bit for bit, what the uninterrupted run gave."""
    recipe = ops.Recipe(format=fmt, amax_history_len=4)
    M, H, F, n, k = 512, 768, 3072, 7, 3
    wl = f"resume/{fmt}"
    full, _ = _mlp_run(recipe, M, H, F, n, 0, None, wl)
    _, snap = _mlp_run(recipe, M, H, F, k, 0, None, wl)
    resumed, _ = _mlp_run(recipe, M, H, F, n, k, snap, wl)
    assert len(resumed) == n - k
    for step, (a, b) in enumerate(zip(full[k:], resumed)):
        for i, (ta, tb) in enumerate(zip(a, b)):
            assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), \
                f"step {k + step}: result {i} differs after resume"
    # the history really carried information: the resumed scales are not fresh ones
    assert not torch.equal(resumed[0][5], torch.ones_like(resumed[0][5]))
