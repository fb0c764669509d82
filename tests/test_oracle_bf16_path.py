"""Pins for the oracle's BF16 (non-FP8) modules (CPU only).

Unit-variance rows of +-1 with gamma = 1, beta = 0 normalise to +-1/sqrt(1 +
eps), which rounds to exactly +-1 in bf16, so on them the modules reduce to
plain integer matrix algebra; permutation weights pin fc2's wiring to torch's
own GELU; random inputs pin the chains against float64 autograd within the
bf16 rounding of the stored activations.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

EPS = 1e-5


def bits(x):
    return oracle.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def unit_rows(M, K, seed):
    """+-1 rows with as many +1 as -1 (mean 0, variance 1)."""
    rng = np.random.default_rng(seed)
    base = np.array([1.0, -1.0] * (K // 2))
    return np.stack([rng.permutation(base) for _ in range(M)])


def test_unit_rows_normalise_to_exact_signs():
    x = unit_rows(8, 64, 1)
    out, ctx = oracle.ln_linear_fwd_bf16(bits(x), bits(np.ones(64)), bits(np.zeros(64)),
                                         bits(np.eye(16, 64)), None, EPS)
    np.testing.assert_array_equal(oracle.bf16_to_f64(ctx["ln_bits"]), x)
    np.testing.assert_array_equal(out, x[:, :16])


def test_bf16_linear_is_exact_integer_algebra_on_unit_rows():
    """out = x W^T + b, dLN = dy W, dW = dy^T x and dbias = sum dy exactly; a
    transposed operand or a dropped term would not match."""
    rng = np.random.default_rng(2)
    M, K, N = 24, 48, 40
    x = unit_rows(M, K, 3)
    w = rng.integers(-4, 5, size=(N, K)) / 4.0
    bias = rng.integers(-8, 9, size=N) / 8.0
    dy = rng.integers(-3, 4, size=(M, N)) / 2.0
    out, ctx = oracle.ln_linear_fwd_bf16(bits(x), bits(np.ones(K)), bits(np.zeros(K)), bits(w),
                                         bits(bias), EPS)
    np.testing.assert_array_equal(out, x @ w.T + bias)
    g = oracle.ln_linear_bwd_bf16(bits(dy), ctx, bits(x), bits(np.ones(K)), bits(w))
    np.testing.assert_array_equal(g["dln"], dy @ w)
    np.testing.assert_array_equal(g["dw"], dy.T @ x)
    np.testing.assert_array_equal(g["dbias"], dy.sum(axis=0))


@pytest.mark.parametrize("act,approx", [(oracle.GELU_TANH, "tanh"), (oracle.GELU_ERF, "none")])
def test_bf16_mlp_fc2_selects_torch_gelu_columns(act, approx):
    """With unit rows, fc1 is exact integer algebra; a selection matrix as W2
    makes out[:, j] = bf16(gelu(h[:, perm[j]])) + b2[j], with gelu from torch."""
    rng = np.random.default_rng(4)
    M, H, Fd = 16, 32, 64
    x = unit_rows(M, H, 5)
    w1 = rng.integers(-2, 3, size=(Fd, H)) / 8.0
    b1 = rng.integers(-4, 5, size=Fd) / 4.0
    perm = rng.permutation(Fd)[:H]
    w2 = np.zeros((H, Fd))
    w2[np.arange(H), perm] = 1.0
    b2 = rng.integers(-4, 5, size=H) / 4.0
    out, ctx = oracle.ln_mlp_fwd_bf16(bits(x), bits(np.ones(H)), bits(np.zeros(H)), bits(w1),
                                      bits(b1), bits(w2), bits(b2), EPS, act)
    h = x @ w1.T + b1
    np.testing.assert_array_equal(ctx["h"], h)
    gt = F.gelu(torch.from_numpy(h), approximate=approx).numpy()
    np.testing.assert_allclose(ctx["g"], gt, rtol=1e-13, atol=1e-15)
    gb = oracle.bf16_to_f64(bits(gt))
    np.testing.assert_array_equal(out, gb[:, perm] + b2)


def _torch_mlp(x, g, b, w1, b1, w2, b2, approx):
    t = lambda a: torch.from_numpy(oracle.bf16_to_f64(a)).requires_grad_()
    xt, w1t, w2t = t(x), t(w1), t(w2)
    y = F.layer_norm(xt, (xt.shape[1],), t(g), t(b), EPS)
    h = y @ w1t.T + t(b1)
    return F.gelu(h, approximate=approx) @ w2t.T + t(b2)


def rel_rows(a, ref):
    return (np.abs(a - ref).max(axis=1) / np.linalg.norm(ref, axis=1)).max()


def test_bf16_linear_tracks_float64_autograd():
    """Random inputs: the chain stays within the bf16 rounding of the LayerNorm
    output (relative 2^-9 per element) of float64 autograd."""
    rng = np.random.default_rng(6)
    M, K, N = 64, 96, 80
    x, g, b = bits(rng.normal(size=(M, K))), bits(1 + 0.1 * rng.normal(size=K)), \
        bits(0.1 * rng.normal(size=K))
    w, bias, dy = bits(0.02 * rng.normal(size=(N, K))), bits(0.1 * rng.normal(size=N)), \
        bits(1e-3 * rng.normal(size=(M, N)))
    out, ctx = oracle.ln_linear_fwd_bf16(x, g, b, w, bias, EPS)
    grads = oracle.ln_linear_bwd_bf16(dy, ctx, x, g, w)
    t = lambda a: torch.from_numpy(oracle.bf16_to_f64(a)).requires_grad_()
    xt, gt, bt, wt, biast = t(x), t(g), t(b), t(w), t(bias)
    ref = F.layer_norm(xt, (K,), gt, bt, EPS) @ wt.T + biast
    ref.backward(torch.from_numpy(oracle.bf16_to_f64(dy)))
    assert rel_rows(out, ref.detach().numpy()) < 4e-3
    assert rel_rows(grads["dw"], wt.grad.numpy()) < 4e-3
    # dLN = dy W takes no rounded operand, so dx, dgamma, dbeta agree closely
    assert rel_rows(grads["dx"], xt.grad.numpy()) < 1e-10
    np.testing.assert_allclose(grads["dgamma"], gt.grad.numpy(), rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(grads["dbeta"], bt.grad.numpy(), rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(grads["dbias"], biast.grad.numpy(), rtol=1e-12, atol=0)


@pytest.mark.parametrize("act,approx", [(oracle.GELU_TANH, "tanh"), (oracle.GELU_ERF, "none")])
def test_bf16_mlp_tracks_float64_autograd(act, approx):
    rng = np.random.default_rng(7)
    M, H, Fd = 48, 64, 128
    x, g, b = bits(rng.normal(size=(M, H))), bits(1 + 0.1 * rng.normal(size=H)), \
        bits(0.1 * rng.normal(size=H))
    w1, b1 = bits(0.1 * rng.normal(size=(Fd, H))), bits(0.1 * rng.normal(size=Fd))
    w2, b2 = bits(0.1 * rng.normal(size=(H, Fd))), bits(0.1 * rng.normal(size=H))
    out, _ = oracle.ln_mlp_fwd_bf16(x, g, b, w1, b1, w2, b2, EPS, act)
    ref = _torch_mlp(x, g, b, w1, b1, w2, b2, approx).detach().numpy()
    assert rel_rows(out, ref) < 8e-3


@pytest.mark.parametrize("act,approx", [(oracle.GELU_TANH, "tanh"), (oracle.GELU_ERF, "none")])
def test_bf16_mlp_backward_tracks_float64_autograd(act, approx):
    """The backward's only roundings are the stored bf16 h (for gelu'), bf16 g
    (fc2's weight gradient) and bf16 dH; the gradients stay within those
    roundings of float64 autograd."""
    rng = np.random.default_rng(8)
    M, H, Fd = 48, 64, 128
    x, g, b = bits(rng.normal(size=(M, H))), bits(1 + 0.1 * rng.normal(size=H)), \
        bits(0.1 * rng.normal(size=H))
    w1, b1 = bits(0.1 * rng.normal(size=(Fd, H))), bits(0.1 * rng.normal(size=Fd))
    w2, b2 = bits(0.1 * rng.normal(size=(H, Fd))), bits(0.1 * rng.normal(size=H))
    dy = bits(1e-2 * rng.normal(size=(M, H)))
    _, ctx = oracle.ln_mlp_fwd_bf16(x, g, b, w1, b1, w2, b2, EPS, act)
    gr = oracle.ln_mlp_bwd_bf16(dy, ctx, x, g, w1, w2, act)
    t = lambda a: torch.from_numpy(oracle.bf16_to_f64(a)).requires_grad_()
    xt, gt, bt, w1t, b1t, w2t, b2t = map(t, (x, g, b, w1, b1, w2, b2))
    y = F.layer_norm(xt, (H,), gt, bt, EPS)
    out = F.gelu(y @ w1t.T + b1t, approximate=approx) @ w2t.T + b2t
    out.backward(torch.from_numpy(oracle.bf16_to_f64(dy)))
    assert rel_rows(gr["dw2"], w2t.grad.numpy()) < 1e-2
    assert rel_rows(gr["dw1"], w1t.grad.numpy()) < 1e-2
    assert rel_rows(gr["dx"], xt.grad.numpy()) < 1e-2
    for got, ref in ((gr["db1"], b1t.grad), (gr["dgamma"], gt.grad), (gr["dbeta"], bt.grad)):
        assert np.linalg.norm(got - ref.numpy()) / np.linalg.norm(ref.numpy()) < 1e-2
    np.testing.assert_allclose(gr["db2"], b2t.grad.numpy(), rtol=1e-12, atol=0)


def test_bf16_mlp_backward_on_unit_rows_with_linear_gelu_region():
    """Large positive h (> 8) puts GELU where gelu(h) = h and gelu'(h) = 1 to far
    below bf16 resolution: the backward is then the plain algebra of two linear
    layers, dH = dy W2 (bf16), dW2 = dy^T g, dW1 = dH^T x."""
    rng = np.random.default_rng(9)
    M, H, Fd = 16, 32, 48
    x = unit_rows(M, H, 10)
    w1 = np.zeros((Fd, H))
    b1 = 8.0 + rng.integers(0, 8, size=Fd)          # h = b1 >= 8 for every row
    w2 = rng.integers(-2, 3, size=(H, Fd)) / 4.0
    dy = rng.integers(-2, 3, size=(M, H)) / 8.0
    args = (bits(x), bits(np.ones(H)), bits(np.zeros(H)), bits(w1), bits(b1), bits(w2),
            bits(np.zeros(H)))
    out, ctx = oracle.ln_mlp_fwd_bf16(*args, EPS)
    np.testing.assert_array_equal(oracle.bf16_to_f64(ctx["g_bits"]), np.tile(b1, (M, 1)))
    gr = oracle.ln_mlp_bwd_bf16(bits(dy), ctx, bits(x), bits(np.ones(H)), bits(w1), bits(w2))
    dh = dy @ w2
    np.testing.assert_array_equal(oracle.bf16_to_f64(gr["dh_bits"]), dh)
    np.testing.assert_array_equal(gr["dw2"], dy.T @ np.tile(b1, (M, 1)))
    np.testing.assert_array_equal(gr["dw1"], dh.T @ x)
    np.testing.assert_array_equal(gr["db1"], dh.sum(axis=0))
