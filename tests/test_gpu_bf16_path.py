"""GPU parity of the BF16 (non-FP8) path: the bf16 MFMA GEMM (bit-exact on
exactly summable inputs, across every tile shape), its GELU epilogue, the bf16
transpose with column sums, and the BF16 LayerNormLinear / LayerNormMLP
modules against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from fp8_delayed_scaling_row_amd import inputs, ops
from parity import (assert_gemm_close, assert_vector_close, compare_bf16, ln_window, to_np,
                    to_np_bits)

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-5))
GELU = {ops.GELU_TANH: oracle.gelu_tanh, ops.GELU_ERF: oracle.gelu_erf}


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def int_bf16(shape, seed, lim=4):
    vals = np.random.default_rng(seed).integers(-lim, lim + 1, size=shape).astype(np.float64)
    return oracle.f64_to_bf16_bits(vals), vals


# (M, N, K): 64 x 64 tiles, 128 x 128, 128 x 256, and 256 x 256 (K > 1024; its steps
# of 32 elements run in rounds of eight, here with 1, 4 and 7 steps over)
SHAPES = [(1, 16, 16), (130, 144, 272), (257, 400, 64), (1024, 1024, 512), (2048, 1024, 128),
          (4096, 4096, 256), (4096, 4096, 1040), (4096, 4096, 1152), (4096, 4096, 1248)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_gemm_is_bit_exact_on_small_integers(M, N, K):
    """|a|, |b| <= 4 and K <= 1248: every partial sum is an integer below 2^24, so
    fp32 accumulation in any order is exact."""
    a, av = int_bf16((M, K), M + 3 * K)
    b, bv = int_bf16((N, K), N + 5 * K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm_bf16(bf16_dev(a), bf16_dev(b), out)
    bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(N).integers(-64, 65, N) / 8.0)
    out16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm_bf16(bf16_dev(a), bf16_dev(b), out16, bias=bf16_dev(bias_bits))
    torch.cuda.synchronize()
    ref = av @ bv.T
    np.testing.assert_array_equal(out.cpu().numpy(), ref)
    ref16 = oracle.f64_to_bf16_bits(ref + oracle.bf16_to_f64(bias_bits)[None, :])
    np.testing.assert_array_equal(to_np_bits(out16), ref16)


def test_bf16_gemm_layout_pins():
    """A permutation as B picks columns of A: C[m][n] = A[m][perm[n]]."""
    M, N, K = 96, 128, 320
    a, av = int_bf16((M, K), 11, lim=100)
    perm = np.random.default_rng(1).permutation(K)[:N]
    bv = np.zeros((N, K))
    bv[np.arange(N), perm] = 1.0
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm_bf16(bf16_dev(a), bf16_dev(oracle.f64_to_bf16_bits(bv)), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), av[:, perm])


@pytest.mark.parametrize("M,N,K", [(300, 272, 96), (2048, 3072, 768)])
def test_bf16_gemm_random_operands(M, N, K):
    rng = np.random.default_rng(M + N)
    a = oracle.f64_to_bf16_bits(rng.normal(size=(M, K)))
    b = oracle.f64_to_bf16_bits(0.02 * rng.normal(size=(N, K)))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm_bf16(bf16_dev(a), bf16_dev(b), out)
    torch.cuda.synchronize()
    assert_gemm_close(out.cpu().numpy(), oracle.gemm_bf16(a, b), tol=1e-5, alarm=1e-5)


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,N,K", [(64, 128, 64), (130, 272, 48), (2048, 3072, 768)])
def test_bf16_gelu_epilogue_on_exact_products(M, N, K, act):
    """Exact h (small integers over 8): h_out matches bit for bit, gelu's bf16
    output matches except where the fp32 GELU's error reaches a midpoint."""
    a, av = int_bf16((M, K), 5 + M, lim=2)
    b, bv = int_bf16((N, K), 7 + N, lim=2)
    bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(N).integers(-64, 65, N) / 64.0)
    b8 = oracle.f64_to_bf16_bits(bv / 8.0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    h_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm_gelu_bf16(bf16_dev(a), bf16_dev(b8), out, bias=bf16_dev(bias_bits), h_out=h_out,
                       activation=act)
    torch.cuda.synchronize()
    h = av @ (bv / 8.0).T + oracle.bf16_to_f64(bias_bits)[None, :]
    np.testing.assert_array_equal(to_np_bits(h_out), oracle.f64_to_bf16_bits(h))
    g = GELU[act](h)
    # the fp32 GELU's error is about 1e-6 of |h| (the exp2 and reciprocal steps):
    # where |g| << |h| (h well below 0) that window spans a good part of a bf16 ulp
    stats = compare_bf16(to_np_bits(out), g, 2e-6 * np.abs(h) + 1e-6 * np.abs(g))
    print(f"gelu bf16 {M}x{N}: {stats}")


@pytest.mark.parametrize("rows,cols", [(8, 8), (64, 64), (200, 136), (2048, 2304), (0, 64)])
def test_bf16_transpose_and_column_sums(rows, cols):
    x = inputs.normal_bf16((rows, cols), inputs.seed_for("tb16", f"{rows}x{cols}"))
    out = torch.empty((cols, rows), dtype=torch.bfloat16, device="cuda")
    cs = torch.full((cols,), float("nan"), dtype=torch.float32, device="cuda")
    xd = x.cuda()
    ops.transpose_bf16(xd, out, cs)
    torch.cuda.synchronize()
    assert torch.equal(out, xd.t().contiguous())
    ref = oracle.bf16_to_f64(to_np_bits(x)).sum(axis=0)
    scale = np.abs(oracle.bf16_to_f64(to_np_bits(x))).sum(axis=0)
    assert np.all(np.abs(cs.cpu().numpy() - ref) <= 1e-6 * scale + 1e-30)


# ---- modules ---------------------------------------------------------------------

def module_inputs(M, K, N, wl):
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x"))
    g, b = inputs.layernorm_params(K, wl)
    w = inputs.linear_weight(N, K, wl, "weight")
    bias = inputs.normal_bf16((N,), inputs.seed_for(wl, "bias"), std=0.1)
    return x, g, b, w, bias


@pytest.mark.parametrize("M,K,N", [(2048, 768, 2304), (48, 64, 80), (144, 256, 400),
                                   (4096, 2048, 2048), (0, 64, 32)])
def test_bf16_ln_linear_fwd_bwd(M, K, N):
    wl = f"bf16lin/{M}/{K}/{N}"
    x, g, b, w, bias = module_inputs(M, K, N, wl)
    dy = inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy"), std=1e-3)
    xd, gd, bd, wd, biasd, dyd = (t.cuda() for t in (x, g, b, w, bias, dy))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ln_out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    ops.ln_linear_fwd_bf16(xd, gd, bd, wd, biasd, out, ln_out, mean, rstd)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dgamma = torch.empty(K, dtype=torch.float32, device="cuda")
    dbeta = torch.empty(K, dtype=torch.float32, device="cuda")
    dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    dbias = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    ops.ln_linear_bwd_bf16(dyd, xd, gd, wd, ln_out, mean, rstd, dx, dgamma, dbeta, dw, dbias)
    torch.cuda.synchronize()
    xb, gb, bb, wb, biasb, dyb = map(to_np_bits, (x, g, b, w, bias, dy))
    oout, octx = oracle.ln_linear_fwd_bf16(xb, gb, bb, wb, biasb, EPS)
    if M == 0:
        assert not dw.any().item() and not dbias.any().item()
        assert not dgamma.any().item() and not dbeta.any().item()
        return
    # the LayerNorm output: the fused LayerNorm's window
    xv, gv, bv = (oracle.bf16_to_f64(t) for t in (xb, gb, bb))
    gx = (xv - octx["mean"][:, None]) * octx["rstd"][:, None] * gv
    compare_bf16(to_np_bits(ln_out), octx["y"], ln_window(gx, bv, 1.0, octx["y"]))
    assert_gemm_close(to_np(out), oout, alarm=5e-3, what="out")
    # identical inputs: the GEMM of the GPU's own LayerNorm output
    gl = to_np_bits(ln_out)
    ref = oracle.gemm_bf16(gl, wb, biasb)
    assert_gemm_close(to_np(out), ref, tol=4e-3, alarm=3e-3, what="out (same ln_out)")
    ctx = dict(ln_bits=gl, mean=mean.cpu().numpy().astype(np.float64),
               rstd=rstd.cpu().numpy().astype(np.float64))
    og = oracle.ln_linear_bwd_bf16(dyb, ctx, xb, gb, wb)
    assert_gemm_close(dw.cpu().numpy(), og["dw"], tol=1e-5, alarm=1e-5, what="dW")
    assert_vector_close(dbias.cpu().numpy(), og["dbias"], 1e-6, "dbias")
    assert_vector_close(dgamma.cpu().numpy(), og["dgamma"], 1e-5, "dgamma")
    assert_vector_close(dbeta.cpu().numpy(), og["dbeta"], 1e-5, "dbeta")
    gdx, odx = to_np(dx), og["dx"]
    norms = np.linalg.norm(odx, axis=1)
    assert np.all(np.abs(gdx - odx).max(axis=1) <= 1e-2 * norms + 1e-30)   # bf16 output


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,H,F", [(2048, 768, 3072), (144, 256, 400), (4096, 2048, 8192)])
def test_bf16_ln_mlp_fwd(M, H, F, act):
    wl = f"bf16mlp/{M}/{H}/{F}"
    x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"))
    g, b = inputs.layernorm_params(H, wl)
    w1 = inputs.linear_weight(F, H, wl, "w1")
    w2 = inputs.linear_weight(H, F, wl, "w2")
    b1 = inputs.normal_bf16((F,), inputs.seed_for(wl, "b1"), std=0.1)
    b2 = inputs.normal_bf16((H,), inputs.seed_for(wl, "b2"), std=0.1)
    d = lambda t: t.cuda()
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ln_out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    hh = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    gg = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    ops.ln_mlp_fwd_bf16(d(x), d(g), d(b), d(w1), d(b1), d(w2), d(b2), out, ln_out, gg, h=hh,
                        activation=act)
    torch.cuda.synchronize()
    xb, gb, bb, w1b, b1b, w2b, b2b = map(to_np_bits, (x, g, b, w1, b1, w2, b2))
    rows = slice(None) if M <= 2048 else np.arange(0, M, 61)   # sampled rows at full size
    oout, octx = oracle.ln_mlp_fwd_bf16(xb[rows], gb, bb, w1b, b1b, w2b, b2b, EPS, act)
    assert_gemm_close(to_np(out)[rows], oout, alarm=5e-3, what="out")
    # identical inputs, stage by stage, from the GPU's own bf16 tensors
    gl = to_np_bits(ln_out)[rows]
    h_ref = oracle.gemm_bf16(gl, w1b, b1b)
    assert_gemm_close(to_np(hh)[rows], h_ref, tol=4e-3, alarm=3e-3, what="h")
    g_ref = GELU[act](h_ref)
    assert_gemm_close(to_np(gg)[rows], g_ref, tol=4e-3, alarm=3e-3, what="g")
    o_ref = oracle.gemm_bf16(to_np_bits(gg)[rows], w2b, b2b)
    assert_gemm_close(to_np(out)[rows], o_ref, tol=4e-3, alarm=3e-3, what="out (same g)")


GELU_GRAD = {ops.GELU_TANH: oracle.gelu_tanh_grad, ops.GELU_ERF: oracle.gelu_erf_grad}


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,N,K", [(64, 128, 64), (130, 272, 48), (2048, 3072, 768)])
def test_bf16_dgelu_epilogue_on_exact_products(M, N, K, act):
    """Exact products times gelu'(h): the bf16 output is the rounding of the
    float64 value except within the fp32 gelu' error (4e-6 of |acc|) of a
    midpoint."""
    a, av = int_bf16((M, K), 9 + M, lim=3)
    b, bv = int_bf16((N, K), 3 + N, lim=3)
    h_bits = oracle.f64_to_bf16_bits(np.random.default_rng(M).normal(size=(M, N)) * 2.0)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm_dgelu_bf16(bf16_dev(a), bf16_dev(b), bf16_dev(h_bits), out, activation=act)
    torch.cuda.synchronize()
    acc = av @ bv.T
    ref = acc * GELU_GRAD[act](oracle.bf16_to_f64(h_bits))
    stats = compare_bf16(to_np_bits(out), ref, 4e-6 * np.abs(acc))
    print(f"dgelu bf16 {M}x{N}: {stats}")


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,H,F", [(2048, 768, 3072), (144, 256, 400), (0, 64, 128)])
def test_bf16_ln_mlp_bwd(M, H, F, act):
    """The BF16 LayerNormMLP backward against the oracle fed the GPU forward's own
    bf16 tensors (ln_out, h, g) and row statistics."""
    wl = f"bf16mlpb/{M}/{H}/{F}"
    x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"))
    g, b = inputs.layernorm_params(H, wl)
    w1 = inputs.linear_weight(F, H, wl, "w1")
    w2 = inputs.linear_weight(H, F, wl, "w2")
    b1 = inputs.normal_bf16((F,), inputs.seed_for(wl, "b1"), std=0.1)
    dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-2)
    d = lambda t: t.cuda()
    f32 = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    out, ln_out, hh, gg = bf(M, H), bf(M, H), bf(M, F), bf(M, F)
    mean, rstd = f32(M), f32(M)
    xd, gd, bd, w1d, w2d = d(x), d(g), d(b), d(w1), d(w2)
    ops.ln_mlp_fwd_bf16(xd, gd, bd, w1d, d(b1), w2d, None, out, ln_out, gg, h=hh, mean=mean,
                        rstd=rstd, activation=act)
    dx = bf(M, H)
    dgamma, dbeta, dw1, db1, dw2, db2 = f32(H), f32(H), f32(F, H), f32(F), f32(H, F), f32(H)
    ops.ln_mlp_bwd_bf16(d(dy), xd, gd, w1d, w2d, ln_out, hh, gg, mean, rstd, dx, dgamma, dbeta,
                        dw1, db1, dw2, db2, activation=act)
    torch.cuda.synchronize()
    if M == 0:
        for t in (dgamma, dbeta, dw1, db1, dw2, db2):
            assert not t.any().item()
        return
    ctx = dict(ln_bits=to_np_bits(ln_out), h_bits=to_np_bits(hh), g_bits=to_np_bits(gg),
               mean=mean.cpu().numpy().astype(np.float64),
               rstd=rstd.cpu().numpy().astype(np.float64))
    og = oracle.ln_mlp_bwd_bf16(to_np_bits(dy), ctx, to_np_bits(x), to_np_bits(g),
                                to_np_bits(w1), to_np_bits(w2), act)
    assert_gemm_close(dw2.cpu().numpy(), og["dw2"], tol=1e-5, alarm=1e-5, what="dW2")
    assert_vector_close(db2.cpu().numpy(), og["db2"], 1e-6, "db2")
    # dH is rounded to bf16 on both sides; a value next to a midpoint may round
    # the other way, which moves the sums below by far less than these bounds
    assert_gemm_close(dw1.cpu().numpy(), og["dw1"], tol=1e-3, alarm=1e-3, what="dW1")
    assert_vector_close(db1.cpu().numpy(), og["db1"], 1e-3, "db1")
    assert_vector_close(dgamma.cpu().numpy(), og["dgamma"], 1e-3, "dgamma")
    assert_vector_close(dbeta.cpu().numpy(), og["dbeta"], 1e-3, "dbeta")
    gdx, odx = to_np(dx), og["dx"]
    norms = np.linalg.norm(odx, axis=1)
    assert np.all(np.abs(gdx - odx).max(axis=1) <= 1e-2 * norms + 1e-30)
