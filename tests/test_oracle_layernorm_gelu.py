"""Pins for the oracle's LayerNorm and GELU (CPU only).

LayerNorm and the tanh GELU reduce to library routines (torch.nn.functional in
float64), which pin the oracle's forms; invariants and finite differences pin
the backward and the derivative independently of any library.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(size=shape) * scale


@pytest.mark.parametrize("H", [8, 768, 2048])
def test_layernorm_matches_torch_float64(H):
    x = rand((37, H), 1, 3.0) + 0.5
    g = 1 + 0.1 * rand(H, 2)
    b = 0.1 * rand(H, 3)
    y, mean, rstd = oracle.layernorm_fwd(x, g, b, 1e-5)
    ref = F.layer_norm(torch.from_numpy(x), (H,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13)


def test_layernorm_unit_affine_gives_zero_mean_unit_variance():
    H = 2048
    x = rand((16, H), 4, 2.0)
    y, _, _ = oracle.layernorm_fwd(x, np.ones(H), np.zeros(H), 1e-5)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-12)


def test_layernorm_constant_row_gives_beta_and_is_scale_invariant():
    H = 64
    b = rand(H, 5)
    y, _, rstd = oracle.layernorm_fwd(np.full((1, H), 3.25), np.ones(H), b, 1e-5)
    np.testing.assert_allclose(y[0], b, atol=0)
    assert rstd[0] == 1 / np.sqrt(1e-5)
    x = rand((4, H), 6)
    y1, _, _ = oracle.layernorm_fwd(x, np.ones(H), np.zeros(H), 0.0)
    y2, _, _ = oracle.layernorm_fwd(x * 1000.0, np.ones(H), np.zeros(H), 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-12)
    # |xhat| <= sqrt(H - 1) for any row
    assert np.abs(y1).max() <= np.sqrt(H - 1) + 1e-12


def test_layernorm_backward_matches_torch_autograd():
    H = 96
    x = rand((11, H), 7)
    g = 1 + 0.1 * rand(H, 8)
    b = 0.1 * rand(H, 9)
    dy = rand((11, H), 10)
    _, mean, rstd = oracle.layernorm_fwd(x, g, b, 1e-5)
    dx, dg, db = oracle.layernorm_bwd(dy, x, g, mean, rstd)
    xt = torch.from_numpy(x).requires_grad_()
    gt = torch.from_numpy(g).requires_grad_()
    bt = torch.from_numpy(b).requires_grad_()
    F.layer_norm(xt, (H,), gt, bt, 1e-5).backward(torch.from_numpy(dy))
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_layernorm_backward_finite_differences_and_invariants():
    H = 12
    x = rand((3, H), 11)
    g = 1 + 0.3 * rand(H, 12)
    b = rand(H, 13)
    dy = rand((3, H), 14)
    _, mean, rstd = oracle.layernorm_fwd(x, g, b, 1e-5)
    dx, dg, db = oracle.layernorm_bwd(dy, x, g, mean, rstd)
    loss = lambda xx: (oracle.layernorm_fwd(xx, g, b, 1e-5)[0] * dy).sum()
    h = 1e-6
    num = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(H):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            num[i, j] = (loss(xp) - loss(xm)) / (2 * h)
    np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dx.sum(axis=1), 0, atol=1e-12)     # sum_k dx = 0 per row
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-14)


def test_gelu_tanh_matches_torch_and_identities():
    h = np.linspace(-12, 12, 20001)
    ref = F.gelu(torch.from_numpy(h), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(h), ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(0.0) == 0.0
    # gelu(x) - gelu(-x) = x  (0.5 x (1 + tanh u) - 0.5 (-x)(1 - tanh u))
    np.testing.assert_allclose(oracle.gelu_tanh(h) - oracle.gelu_tanh(-h), h, atol=1e-13)
    # asymptotes: x for large positive, 0 for large negative
    assert abs(oracle.gelu_tanh(30.0) - 30.0) < 1e-12 and abs(oracle.gelu_tanh(-30.0)) < 1e-12
    # close to the erf form everywhere
    erf = F.gelu(torch.from_numpy(h)).numpy()
    assert np.abs(oracle.gelu_tanh(h) - erf).max() < 1e-3


def test_gelu_tanh_grad_matches_finite_differences_and_autograd():
    h = np.linspace(-8, 8, 4001)
    d = 1e-6
    num = (oracle.gelu_tanh(h + d) - oracle.gelu_tanh(h - d)) / (2 * d)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(h), num, rtol=1e-7, atol=1e-9)
    ht = torch.from_numpy(h).requires_grad_()
    F.gelu(ht, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_tanh_grad(h), ht.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_gelu_erf_matches_torch_and_identities():
    h = np.linspace(-12.0, 12.0, 4801)
    ref = F.gelu(torch.from_numpy(h)).numpy()             # the exact erf form
    np.testing.assert_allclose(oracle.gelu_erf(h), ref, rtol=1e-14, atol=1e-15)
    # gelu(x) - gelu(-x) = x, since erf is odd
    np.testing.assert_allclose(oracle.gelu_erf(h) - oracle.gelu_erf(-h), h, atol=1e-13)
    assert oracle.gelu_erf(0.0) == 0.0
    assert abs(oracle.gelu_erf(30.0) - 30.0) < 1e-12 and abs(oracle.gelu_erf(-30.0)) < 1e-12
    # Phi(1) = 0.841344746068543 (standard normal CDF at 1): gelu(1) = Phi(1)
    assert abs(float(oracle.gelu_erf(1.0)) - 0.841344746068543) < 1e-14


def test_gelu_erf_grad_matches_finite_differences_and_autograd():
    h = np.linspace(-9.0, 9.0, 3601)
    d = 1e-6
    num = (oracle.gelu_erf(h + d) - oracle.gelu_erf(h - d)) / (2 * d)
    np.testing.assert_allclose(oracle.gelu_erf_grad(h), num, rtol=1e-7, atol=1e-9)
    ht = torch.from_numpy(h.copy()).requires_grad_(True)
    F.gelu(ht).sum().backward()
    np.testing.assert_allclose(oracle.gelu_erf_grad(h), ht.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_layernorm_module_rounds_the_float64_result_once():
    """The plain LayerNorm module's bf16 output is one nearest-even rounding of
    the float64 LayerNorm: it matches torch's float64 layer_norm converted to
    bf16 through float32 wherever that double rounding is harmless, i.e. the
    float64 value is not within a float32 ulp of a bf16 midpoint."""
    rng = np.random.default_rng(5)
    H = 96
    x = oracle.f64_to_bf16_bits(rng.normal(1.0, 3.0, size=(40, H)))
    g = oracle.f64_to_bf16_bits(1 + 0.1 * rng.normal(size=H))
    b = oracle.f64_to_bf16_bits(0.1 * rng.normal(size=H))
    out = oracle.layernorm(x, g, b, 1e-5)
    t = lambda bits: torch.from_numpy(oracle.bf16_to_f64(bits))
    ref = F.layer_norm(t(x), (H,), t(g), t(b), 1e-5)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    tb = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (out["y_bits"] == tb).mean() > 0.999
    assert np.all(np.abs(oracle.bf16_to_f64(out["y_bits"]) - ref.numpy())
                  <= 2.0 ** -8 * np.abs(ref.numpy()))
