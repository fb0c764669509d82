"""GPU parity: the FP8 MFMA GEMM (bit-exact on exactly summable inputs, layout
pins, and the oracle tolerance on random operands and ragged shapes)."""
import numpy as np
import pytest
import torch

import oracle
from fp8_delayed_scaling_row_amd import ops
from parity import assert_gemm_close, to_np

pytestmark = pytest.mark.gpu

FMT = {ops.E4M3: oracle.E4M3, ops.E5M2: oracle.E5M2}
PAIRS = [(ops.E4M3, ops.E4M3), (ops.E5M2, ops.E4M3), (ops.E4M3, ops.E5M2), (ops.E5M2, ops.E5M2)]


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def int_codes(shape, fp8, seed, lim=8):
    """Codes of small integers in [-lim, lim] (exact in both formats)."""
    vals = np.random.default_rng(seed).integers(-lim, lim + 1, size=shape).astype(np.float64)
    return oracle.fp8_encode(vals, FMT[fp8]), vals


def finite_codes(shape, fp8, seed):
    t = oracle.fp8_decode_table(FMT[fp8])
    fin = np.array([c for c in range(256) if np.isfinite(t[c])], dtype=np.uint8)
    return np.random.default_rng(seed).choice(fin, size=shape)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("fa,fb", PAIRS, ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (128, 128, 256), (130, 144, 272), (1, 16, 16),
                                   (257, 400, 64), (96, 208, 1024)])
def test_small_integer_gemm_is_bit_exact(fa, fb, M, N, K):
    """|a|, |b| <= 8 and K <= 1024: every partial sum is an integer below 2^24, so
    fp32 accumulation in any order is exact."""
    a, av = int_codes((M, K), fa, M * 7 + K)
    b, bv = int_codes((N, K), fb, N * 3 + K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(1.0), _scalar(1.0), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), av @ bv.T)


# Small products on 64 x 64 tiles with 1, 16, 49, 33, 23 and 17 steps of K
# (whole rounds of the four-stage ring with 0, 1 and 3 steps over), the last cut
# on every edge (M % 64, N % 64 and K % 64 all 16).
@pytest.mark.parametrize("fa,fb", PAIRS, ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (200, 144, 1024), (1024, 512, 3136),
                                   (130, 208, 2112), (70, 64, 1472), (2000, 784, 1040)])
def test_small_tile_variants_are_bit_exact(fa, fb, M, N, K):
    """|a|, |b| <= 8 and K <= 3136: every partial sum is an integer below 2^24."""
    a, av = int_codes((M, K), fa, M * 5 + K)
    b, bv = int_codes((N, K), fb, N * 11 + K)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(1.0), _scalar(1.0), out)
    bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(N).integers(-64, 65, N) / 64.0)
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ob = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(0.5), _scalar(0.25), ob, bias)
    torch.cuda.synchronize()
    exact = av @ bv.T
    np.testing.assert_array_equal(out.cpu().numpy(), exact)
    ref = oracle.f64_to_bf16_bits(exact * 0.125 + oracle.bf16_to_f64(bias_bits)[None, :])
    np.testing.assert_array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), ref)


def test_layout_pins_permutation_and_single_entries():
    M, N, K = 64, 128, 256
    rng = np.random.default_rng(0)
    a, av = int_codes((M, K), ops.E4M3, 1)
    perm = rng.permutation(K)[:N]
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), perm] = 0x38                        # 1.0: column n picks k = perm[n]
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm(dev(a), ops.E4M3, dev(b), ops.E4M3, _scalar(1.0), _scalar(1.0), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), av[:, perm])
    # one non-zero product: A[i][k] = 2, B[j][k] = 3 -> C[i][j] = 6 only
    for (i, j, k) in [(0, 0, 0), (63, 127, 255), (17, 33, 129), (5, 100, 31)]:
        a = np.zeros((M, K), dtype=np.uint8)
        b = np.zeros((N, K), dtype=np.uint8)
        a[i, k] = oracle.fp8_encode(2.0, oracle.E4M3)
        b[j, k] = oracle.fp8_encode(3.0, oracle.E4M3)
        ops.gemm(dev(a), ops.E4M3, dev(b), ops.E4M3, _scalar(1.0), _scalar(1.0), out)
        torch.cuda.synchronize()
        expect = np.zeros((M, N))
        expect[i, j] = 6.0
        np.testing.assert_array_equal(out.cpu().numpy(), expect)


@pytest.mark.parametrize("fa,fb", PAIRS[:3], ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2"])
@pytest.mark.parametrize("M,N,K,out_bf16", [
    (256, 2304, 768, True),       # LayerNormLinear forward, batch 8 x 32
    (2048, 768, 3072, True),      # fc2 of the LayerNormMLP
    (333, 272, 528, True),        # ragged M, several tiles
    (2304, 768, 2048, False),     # wgrad shape
    (77, 48, 16, False),
])
def test_random_gemm_within_tolerance(fa, fb, M, N, K, out_bf16):
    a = finite_codes((M, K), fa, 11 + M)
    b = finite_codes((N, K), fb, 13 + N)
    sa, sb = np.float32(1.0 / 37.0), np.float32(1.0 / 1536.0)
    bias = None
    bias_bits = None
    if out_bf16:
        bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(3).normal(size=N) * 50.0)
        bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((M, N), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(float(sa)), _scalar(float(sb)), out, bias)
    torch.cuda.synchronize()
    ref = oracle.fp8_gemm_tn(a, FMT[fa], b, FMT[fb], sa, sb,
                             None if bias_bits is None else oracle.bf16_to_f64(bias_bits))
    # bf16 output rounding alone is 2^-9 relative per element
    # operands are given as codes, so only accumulation and output rounding differ
    assert_gemm_close(to_np(out), ref, alarm=5e-3 if out_bf16 else 1e-3)


def test_k_zero_gives_bias_and_m_zero_is_a_no_op():
    N = 32
    bias_bits = oracle.f64_to_bf16_bits(np.arange(N, dtype=np.float64))
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((4, N), 9.0, dtype=torch.bfloat16, device="cuda")
    a = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    b = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    ops.gemm(a, ops.E4M3, b, ops.E4M3, _scalar(1.0), _scalar(1.0), out, bias)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out), np.tile(np.arange(N, dtype=np.float64), (4, 1)))
    out0 = torch.empty((0, N), dtype=torch.float32, device="cuda")
    ops.gemm(torch.empty((0, 64), dtype=torch.uint8, device="cuda"), ops.E4M3,
             torch.zeros((N, 64), dtype=torch.uint8, device="cuda"), ops.E4M3, _scalar(1.0),
             _scalar(1.0), out0)
    torch.cuda.synchronize()


def test_gemm_is_deterministic():
    M, N, K = 512, 768, 2048
    a = dev(finite_codes((M, K), ops.E4M3, 1))
    b = dev(finite_codes((N, K), ops.E4M3, 2))
    o1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    ops.gemm(a, ops.E4M3, b, ops.E4M3, _scalar(0.5), _scalar(0.25), o1)
    ops.gemm(a, ops.E4M3, b, ops.E4M3, _scalar(0.5), _scalar(0.25), o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---- the MLP epilogues, pinned on exactly representable GEMM results -----------

GELU_REL = 2e-6     # fp32 GELU (tanh via exp): ~1e-6 of |h| plus a few ulps of g


GELU = {ops.GELU_TANH: (oracle.gelu_tanh, oracle.gelu_tanh_grad),
        ops.GELU_ERF: (oracle.gelu_erf, oracle.gelu_erf_grad)}


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,N,K,q", [(64, 128, 64, ops.E4M3), (130, 272, 48, ops.E5M2),
                                     (256, 3072, 32, ops.E4M3)])
def test_gelu_epilogue_on_exact_products(M, N, K, q, act):
    gelu_exact_case(M, N, K, q, act)


def gelu_exact_case(M, N, K, q, act):
    """Small integer operands and power-of-two scale_inv make every h exact in
    fp32, so h (bf16) must match bit for bit and the GELU codes may differ only
    where the fp32 GELU's own error reaches a rounding midpoint."""
    a, av = int_codes((M, K), ops.E4M3, 5 + M, lim=4)
    b, bv = int_codes((N, K), ops.E4M3, 7 + N, lim=4)
    bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(N).integers(-64, 65, N) / 64.0)
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).cuda()
    sa, sb, qs = 1.0 / 16.0, 1.0 / 4.0, float(np.float32(448.0 / 7.3))
    q_out = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    q_t = torch.empty((N, M), dtype=torch.uint8, device="cuda") if M % 16 == 0 else None
    h_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.gemm_gelu_fp8(dev(a), ops.E4M3, dev(b), ops.E4M3, _scalar(sa), _scalar(sb), q,
                      _scalar(qs), amax.data_ptr(), q_out, q_t, h_out, bias, activation=act)
    torch.cuda.synchronize()
    h = (av @ bv.T) * sa * sb + oracle.bf16_to_f64(bias_bits)[None, :]
    np.testing.assert_array_equal(to_np(h_out), oracle.bf16_to_f64(oracle.f64_to_bf16_bits(h)))
    g = GELU[act][0](h)
    fmt = FMT[q]
    from parity import compare_codes
    stats = compare_codes(q_out.cpu().numpy(), g * qs, fmt,
                          qs * (GELU_REL * np.abs(h) + 1e-6 * np.abs(g)))
    assert stats["mismatched"] <= max(2, stats["n"] // 10000), stats
    oamax = float(np.abs(g).max())
    assert abs(amax.item() - oamax) <= 1e-5 * oamax
    if q_t is not None:
        assert torch.equal(q_t, q_out.t().contiguous())


@pytest.mark.parametrize("act", [ops.GELU_TANH, ops.GELU_ERF], ids=["tanh", "erf"])
@pytest.mark.parametrize("M,N,K", [(64, 128, 64), (130, 272, 48)])
def test_dgelu_epilogue_on_exact_products(M, N, K, act):
    a, av = int_codes((M, K), ops.E5M2, 9 + M, lim=4)
    b, bv = int_codes((N, K), ops.E4M3, 3 + N, lim=4)
    h_bits = oracle.f64_to_bf16_bits(np.random.default_rng(M).normal(size=(M, N)) * 2.0)
    h = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sa, sb = 1.0 / 8.0, 2.0
    ops.gemm_dgelu(dev(a), ops.E5M2, dev(b), ops.E4M3, _scalar(sa), _scalar(sb), h, out,
                   activation=act)
    torch.cuda.synchronize()
    acc = (av @ bv.T) * sa * sb
    ref = acc * GELU[act][1](oracle.bf16_to_f64(h_bits))
    err = np.abs(out.cpu().numpy() - ref)
    assert np.all(err <= 4e-6 * np.abs(acc) + 1e-30), err.max()


@pytest.mark.parametrize("M,N,K", [(2048, 3072, 768), (333, 400, 272)])
def test_gelu_gemm_random_within_tolerance(M, N, K):
    """Gaussian-like operands: h under the GEMM rule, the GELU codes within the
    GEMM's error bound carried through GELU'."""
    rng = np.random.default_rng(K)
    a = oracle.fp8_encode(rng.normal(size=(M, K)) * 60, oracle.E4M3)
    b = oracle.fp8_encode(rng.normal(size=(N, K)) * 90, oracle.E4M3)
    sa, sb = np.float32(1 / 60.0), np.float32(1 / 4500.0)
    qs = np.float32(448.0 / 3.0)
    q_out = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    h_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.gemm_gelu_fp8(dev(a), ops.E4M3, dev(b), ops.E4M3, _scalar(float(sa)), _scalar(float(sb)),
                      ops.E4M3, _scalar(float(qs)), amax.data_ptr(), q_out, None, h_out)
    torch.cuda.synchronize()
    h = oracle.fp8_gemm_tn(a, oracle.E4M3, b, oracle.E4M3, sa, sb)
    assert_gemm_close(to_np(h_out), h, alarm=5e-3)
    abs_sum = oracle.fp8_gemm_tn(a & 0x7F, oracle.E4M3, b & 0x7F, oracle.E4M3, sa, sb)
    dh = 2.0 ** -10 * abs_sum + 2.0 ** -22 * np.abs(h)
    g = oracle.gelu_tanh(h)
    from parity import compare_codes
    win = float(qs) * (np.abs(oracle.gelu_tanh_grad(h)) * dh + GELU_REL * np.abs(h) +
                       1e-6 * np.abs(g))
    stats = compare_codes(q_out.cpu().numpy(), g * float(qs), oracle.E4M3, win)
    print(f"gelu gemm {M}x{N}x{K}: {stats}")


# ---- the large-tile kernel (at least 256 output tiles of 256 x 256) -------------

# 128 x 256 tiles (K <= 2048; the second is ragged in M and N), then 256 x 256
# tiles (K > 2048)
# K steps of 64 bytes left after whole unrolled rounds: the 256 x 256 tile runs
# its steps in rounds of eight (four ring stages, two fragment sets), here with 2,
# 1 and 3 steps over; 128 x 256 tiles (three stages) with 1 and 2
BIG = [(4096, 4096, 64), (4000, 4112, 48), (2048, 8192, 2176), (2048, 8192, 2112),
       (2048, 8192, 2240), (4096, 4096, 320)]
# the 256 x 256 tile with 4, 6 and 7 steps over its rounds of eight
BIG_TAILS = [(2048, 8192, 2304), (2048, 8192, 2432), (2048, 8192, 2496)]


@pytest.mark.parametrize("fa,fb", PAIRS, ids=["e4m3xe4m3", "e5m2xe4m3", "e4m3xe5m2", "e5m2xe5m2"])
@pytest.mark.parametrize("M,N,K", BIG + BIG_TAILS)
def test_small_integer_gemm_large_tiles_is_bit_exact(fa, fb, M, N, K):
    """Exact integer products through the 256 x 256 kernel: fp32 output bit for
    bit, and bf16 output (with a bias on a 1/64 grid) equal to the round-to-
    nearest-even of the exact value."""
    a, av = int_codes((M, K), fa, M + K)
    b, bv = int_codes((N, K), fb, N + 2 * K)
    exact = av @ bv.T
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(1.0), _scalar(1.0), out)
    bias_bits = oracle.f64_to_bf16_bits(np.random.default_rng(N).integers(-64, 65, N) / 64.0)
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ob = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.gemm(dev(a), fa, dev(b), fb, _scalar(0.5), _scalar(0.25), ob, bias)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), exact)
    ref = oracle.f64_to_bf16_bits(exact * 0.125 + oracle.bf16_to_f64(bias_bits)[None, :])
    np.testing.assert_array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("M,N,K", BIG)
def test_gelu_epilogue_large_tiles_on_exact_products(M, N, K):
    gelu_exact_case(M, N, K, ops.E4M3, ops.GELU_TANH)
    gelu_exact_case(M, N, K, ops.E4M3, ops.GELU_ERF)


# ---- fc2 dgrad with the fc1 gradient cast fused ---------------------------------

@pytest.mark.parametrize("M,N,K,q,act", [(130, 272, 48, ops.E5M2, ops.GELU_TANH),
                                         (256, 3072, 64, ops.E5M2, ops.GELU_ERF),
                                         (4096, 4096, 64, ops.E5M2, ops.GELU_TANH),
                                         (4000, 4112, 48, ops.E4M3, ops.GELU_ERF),
                                         (2048, 8192, 2176, ops.E5M2, ops.GELU_TANH)])
def test_dgelu_fp8_epilogue_equals_dgelu_then_cast(M, N, K, q, act):
    """The fused epilogue computes the same fp32 d = acc * alpha * gelu'(h) as the
    fp32 epilogue and casts it like the cast kernel: codes, transpose and amax
    agree bit for bit; the bias gradient (summed in another order) to fp32
    rounding, and it is the same on every run."""
    a = dev(finite_codes((M, K), ops.E5M2, 21 + M))
    b = dev(finite_codes((N, K), ops.E4M3, 22 + N))
    h_bits = oracle.f64_to_bf16_bits(np.random.default_rng(M + N).normal(size=(M, N)) * 2.0)
    h = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).cuda()
    sa, sb = _scalar(1.0 / 3000.0), _scalar(1.0 / 700.0)
    scale = _scalar(float(np.float32(57344.0 / 9.0)) if q == ops.E5M2 else 448.0 / 9.0)
    has_t = M % 16 == 0

    d = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ops.gemm_dgelu(a, ops.E5M2, b, ops.E4M3, sa, sb, h, d, activation=act)
    q1 = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    q1t = torch.empty((N, M), dtype=torch.uint8, device="cuda") if has_t else None
    amax1 = torch.zeros(1, dtype=torch.float32, device="cuda")
    db1 = torch.empty(N, dtype=torch.float32, device="cuda")
    ops.cast_amax(d, q, scale, amax1.data_ptr(), q1, q1t, db1)

    runs = []
    for _ in range(2):
        q2 = torch.empty((M, N), dtype=torch.uint8, device="cuda")
        q2t = torch.empty((N, M), dtype=torch.uint8, device="cuda") if has_t else None
        amax2 = torch.zeros(1, dtype=torch.float32, device="cuda")
        db2 = torch.empty(N, dtype=torch.float32, device="cuda")
        ops.gemm_dgelu_fp8(a, ops.E5M2, b, ops.E4M3, sa, sb, h, q, scale, amax2.data_ptr(), q2,
                           q2t, db2, activation=act)
        runs.append((q2, q2t, amax2, db2))
    torch.cuda.synchronize()
    q2, q2t, amax2, db2 = runs[0]
    assert torch.equal(q1, q2)
    if has_t:
        assert torch.equal(q1t, q2t)
        assert torch.equal(q2t, q2.t().contiguous())
    assert amax1.item() == amax2.item() and amax2.item() > 0
    dsum = d.abs().sum(dim=0)
    assert torch.all((db1 - db2).abs() <= 2e-6 * dsum + 1e-30)
    assert torch.equal(runs[1][3], db2) and torch.equal(runs[1][0], q2)


def _device_finite_codes(shape, fp8, seed):
    """Full-range random finite codes of both signs, drawn on the device."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    c = torch.randint(0, 256, shape, generator=g, dtype=torch.int32, device="cuda")
    bad = (c & 0x7F) == 0x7F if fp8 == ops.E4M3 else (c & 0x7C) == 0x7C
    return torch.where(bad, c & 0x80, c).to(torch.uint8)


@pytest.mark.parametrize("fa,fb", [(ops.E4M3, ops.E4M3), (ops.E5M2, ops.E4M3)],
                         ids=["fc1_e4m3xe4m3", "fc2_dgrad_e5m2xe4m3"])
def test_mfma_dot_product_error_bound(fa, fb):
    """The bound the GEMM-fed code windows rest on, asserted element by element:
    on full-range random codes at the scale-up layer's 16384 x 8192 x 2048 shape
    (fc1; fc2's dgrad with E5M2 gradients), every fp32 output is within
        (2^-10 + (K / 64) 2^-24) sum_k |a b| + 2^-24 |C|
    of the exact product (C++ oracle, integer-accumulated): one FP8 MFMA returns
    its dot product to 2^-10 of its sum of |a b|, the fp32 adds between the K / 64
    instructions round once each, and the result is rounded once."""
    import oracle.cxx as X
    M, N, K = 16384, 8192, 2048
    a = _device_finite_codes((M, K), fa, 101)
    b = _device_finite_codes((N, K), fb, 102)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    one = _scalar(1.0)
    ops.gemm(a, fa, b, fb, one, one, out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(7).integers(0, M, 22)]))
    rt = torch.from_numpy(rows).cuda()
    an, bn = a[rt].cpu().numpy(), b.cpu().numpy()
    exact = X.fp8_gemm_tn(an, FMT[fa], bn, FMT[fb])
    abs_sum = X.fp8_gemm_tn(an & 0x7F, FMT[fa], bn & 0x7F, FMT[fb])
    got = out[rt].cpu().numpy().astype(np.float64)
    err = np.abs(got - exact)
    bound = (2.0 ** -10 + (K / 64) * 2.0 ** -24) * abs_sum + 2.0 ** -24 * np.abs(exact)
    worst = float((err / abs_sum).max())
    print(f"{FMT[fa]} x {FMT[fb]}: max |err| / sum|ab| = {worst:.3e} (bound 2^-10 = 9.8e-4)")
    assert np.all(err <= bound), f"{int((err > bound).sum())} outputs past the bound"
