"""Exact pins for the oracle's FP8 LayerNormLinear and LayerNormMLP chains (CPU).

The chains are checked on inputs built so that every result reduces to exact
dyadic algebra that this file writes out from the readings alone, without the
oracle's encoder or GEMM:

* x rows hold equally many +1 and -1 entries, gamma = 1 and beta = 0: every
  row has mean 0 and variance 1, so the LayerNorm output is +-r with
  r = 1/sqrt(1 + eps), and its FP8 code is exactly +-1 (times the slot's scale);
* weights and output gradients are bf16 values of the binade [1, 2) on a 1/64
  grid, which no FP8 format holds, so every cast really rounds;
* every scale is a power of two (set through the amax history), so a cast of
  v is scale-free: q(v) = RNE of v to the format's significand bits, and a
  wrong scale_inv anywhere is off by a power of two;
* the fc1 bias puts h = fc1 output at 8 or more for the tanh form (24 or
  more for the erf form), where float64 GELU(h) = h and GELU'(h) = 1 exactly,
  while h itself lies between the FP8 values, so the GELU output's cast rounds.

Which operand each product takes is the reading to pin ("Turbo-charging your
transformer training", "Playing with lower-precision formats: BF16 vs FP8":
activations are cast to FP8 with the scaling and the gradients handed back in
BF16/FP32; the wgrad and dgrad products are FP8 products): wgrad multiplies the
FP8 gradient with the forward's saved FP8 activation (LN output, GELU output),
dgrad with the forward's FP8 weight, and bias gradients are column sums of the
unquantised gradient (bf16 dy, float64 dH).  Each alternative reading moves a
result by far more than float64 rounding: the mutation tests at the end plant
them in a copy of the oracle and require the pins to fail.
"""
import inspect
import sys
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.modules
from oracle import E4M3, E5M2

MBITS = {E4M3: 3, E5M2: 2}
MIN_NORMAL = {E4M3: 2.0 ** -6, E5M2: 2.0 ** -14}
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def rne(v, fmt):
    """v rounded to the format's significand (round to nearest, ties to even),
    for values in the format's normal range: with v = f 2^e (0.5 <= |f| < 1)
    the spacing is 2^(e - 1 - mantissa bits)."""
    v = np.asarray(v, dtype=np.float64)
    nz = v != 0
    assert np.all(np.abs(v[nz]) >= MIN_NORMAL[fmt]), "pin input left the normal range"
    _, e = np.frexp(v)
    q = e - 1 - MBITS[fmt]
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    assert np.all(np.abs(r) <= FMAX[fmt]), "pin input saturates"
    return np.where(nz, r, 0.0)


def bits(v):
    return oracle.f64_to_bf16_bits(np.asarray(v, dtype=np.float64))


def exact_bf16(v):
    b = bits(v)
    assert np.array_equal(oracle.bf16_to_f64(b), v), "pin value is not a bf16 value"
    return b


def unit_rows(M, K, rng):
    """M rows of K/2 entries +1 and K/2 entries -1 (mean 0, variance 1)."""
    x = np.ones((M, K))
    for m in range(M):
        x[m, rng.permutation(K)[: K // 2]] = -1.0
    return x


def binade_values(shape, rng, density=1.0):
    """+-[1, 2) on a 1/64 grid (bf16 values that no FP8 format holds when
    off the FP8 grid), a fraction `density` of them non-zero."""
    v = (1.0 + rng.integers(0, 64, size=shape) / 64.0) * rng.choice([-1.0, 1.0], size=shape)
    if density < 1.0:
        v = v * (rng.random(size=shape) < density)
    return v


def k_nonzero_rows(R, C, k, rng):
    """[R][C] with exactly k entries of +-[1, 2) per row."""
    w = np.zeros((R, C))
    for r in range(R):
        idx = rng.permutation(C)[:k]
        w[r, idx] = binade_values(k, rng)
    return w


def set_power_of_two_scales(meta, exps):
    """History row 0 := fp8_max / 2^e per slot, then the step-start update: the
    slot scales become exactly 2^e (and the history rolls, leaving row 0 at 0)."""
    for s, e in enumerate(exps):
        meta.history[0, s] = np.float32(oracle.fp8_max_for(meta.formats[s]) / 2.0 ** e)
    oracle.scaling_update(meta)
    for s, e in enumerate(exps):
        assert meta.scale[s] == np.float32(2.0 ** e)
        assert meta.scale_inv[s] == np.float32(2.0 ** -e)


def dec(codes, fmt, sinv):
    return oracle.fp8_decode(codes, fmt) * float(sinv)


def ln_bwd_reference(dln, x, eps):
    """dx of LayerNorm(x; gamma = 1, beta = 0) for the incoming gradient dln:
    float64 autograd of torch's layer_norm."""
    xt = torch.from_numpy(x).requires_grad_()
    y = F.layer_norm(xt, (x.shape[1],), None, None, eps)
    y.backward(torch.from_numpy(dln))
    return xt.grad.numpy()


FORMATS = [oracle.FORMAT_HYBRID, oracle.FORMAT_E4M3, oracle.FORMAT_E5M2]


# ---- LayerNormLinear -----------------------------------------------------------

def linear_case(seed=0, M=32, K=64, N=48):
    rng = np.random.default_rng(seed)
    x = unit_rows(M, K, rng)
    w = binade_values((N, K), rng)
    bias = np.round(rng.normal(size=N) * 8) / 8
    dy = binade_values((M, N), rng)
    return x, w, bias, dy


def check_ln_linear_pins(om, fmt):
    """Runs one LayerNormLinear step of module implementation `om` on the pin
    inputs and asserts every result against the exact algebra."""
    r = om.Recipe(format=fmt)
    ffmt, bfmt = om.fwd_format(r), om.bwd_format(r)
    x, w, bias, dy = linear_case()
    M, K = x.shape
    eps = r.eps64
    rs = 1.0 / np.sqrt(1.0 + eps)                      # |LN output|
    mf, mb = om.linear_fwd_meta(r), om.linear_bwd_meta(r)
    set_power_of_two_scales(mf, [1, 2])
    set_power_of_two_scales(mb, [3])
    ones, zeros = exact_bf16(np.ones(K)), exact_bf16(np.zeros(K))
    out, ctx = om.ln_linear_fwd(r, mf, exact_bf16(x), ones, zeros, exact_bf16(w),
                                exact_bf16(bias))
    g = om.ln_linear_bwd(r, mf, mb, exact_bf16(dy), ctx, exact_bf16(x), ones)

    w_q = rne(w, ffmt)
    dy_q = rne(dy, bfmt)
    # forward: LN codes are exactly +-1 (in value), the weight rounds
    np.testing.assert_array_equal(dec(ctx["ln_q"], ffmt, mf.scale_inv[0]), x)
    np.testing.assert_array_equal(dec(ctx["w_q"], ffmt, mf.scale_inv[1]), w_q)
    np.testing.assert_array_equal(out, x @ w_q.T + bias)
    assert mf.history[0, 0] == np.float32(rs)
    assert mf.history[0, 1] == np.float32(np.abs(w).max())
    # backward: dgrad on the FP8 weight, wgrad on the saved FP8 LN output,
    # dbias from the unquantised dy
    dln = dy_q @ w_q
    np.testing.assert_array_equal(g["dln"], dln)
    np.testing.assert_array_equal(g["dw"], dy_q.T @ x)
    np.testing.assert_array_equal(g["dbias"], dy.sum(axis=0))
    assert mb.history[0, 0] == np.float32(np.abs(dy).max())
    np.testing.assert_array_equal(g["dbeta"], dln.sum(axis=0))
    np.testing.assert_allclose(g["dgamma"], (dln * x).sum(axis=0) * rs, rtol=1e-14,
                               atol=1e-14 * np.abs(dln).sum(axis=0).max())
    np.testing.assert_allclose(g["dx"], ln_bwd_reference(dln, x, eps), rtol=1e-12,
                               atol=1e-12 * np.abs(dln).max())


@pytest.mark.parametrize("fmt", FORMATS)
def test_ln_linear_chain_exact(fmt):
    check_ln_linear_pins(oracle.modules, fmt)


# ---- Linear (no LayerNorm) -----------------------------------------------------

def check_linear_pins(om, fmt):
    """Linear: the input itself is slot 0, so x, W and dy all round; wgrad
    takes the FP8 input codes."""
    r = om.Recipe(format=fmt)
    ffmt, bfmt = om.fwd_format(r), om.bwd_format(r)
    rng = np.random.default_rng(5)
    M, K, N = 32, 48, 40
    x, w, dy = binade_values((M, K), rng), binade_values((N, K), rng), binade_values((M, N), rng)
    bias = np.round(rng.normal(size=N) * 8) / 8
    mf, mb = om.linear_fwd_meta(r), om.linear_bwd_meta(r)
    set_power_of_two_scales(mf, [2, -1])
    set_power_of_two_scales(mb, [1])
    out, ctx = om.linear_fwd(r, mf, exact_bf16(x), exact_bf16(w), exact_bf16(bias))
    g = om.linear_bwd(r, mf, mb, exact_bf16(dy), ctx)
    x_q, w_q, dy_q = rne(x, ffmt), rne(w, ffmt), rne(dy, bfmt)
    np.testing.assert_array_equal(out, x_q @ w_q.T + bias)
    np.testing.assert_array_equal(g["dx"], dy_q @ w_q)
    np.testing.assert_array_equal(g["dw"], dy_q.T @ x_q)
    np.testing.assert_array_equal(g["dbias"], dy.sum(axis=0))
    assert mf.history[0, 0] == np.float32(np.abs(x).max())
    assert mf.history[0, 1] == np.float32(np.abs(w).max())
    assert mb.history[0, 0] == np.float32(np.abs(dy).max())


@pytest.mark.parametrize("fmt", FORMATS)
def test_linear_chain_exact(fmt):
    check_linear_pins(oracle.modules, fmt)


# ---- LayerNormMLP --------------------------------------------------------------

def mlp_case(activation, seed=1, M=32, H=32, Fd=64):
    rng = np.random.default_rng(seed)
    x = unit_rows(M, H, rng)
    # h = x . w1^T + b1 stays on the bf16 grid: |x . w1| <= 4 and h in [8, 17)
    # for the tanh form; |x . w1| <= 2 and h in [24, 29) for the erf form
    tanh = activation == oracle.GELU_TANH
    w1 = k_nonzero_rows(Fd, H, 2 if tanh else 1, rng)
    b1 = (12.0 if tanh else 26.0) + rng.integers(0, 8, size=Fd) / 8.0
    w2 = k_nonzero_rows(Fd, H, 2, rng).T.copy()        # [H][F], two entries per column
    b2 = np.round(rng.normal(size=H) * 8) / 8
    dy = binade_values((M, H), rng)
    return x, w1, b1, w2, b2, dy


def check_ln_mlp_pins(om, fmt, activation=oracle.GELU_TANH):
    r = om.Recipe(format=fmt, activation=activation)
    ffmt, bfmt = om.fwd_format(r), om.bwd_format(r)
    x, w1, b1, w2, b2, dy = mlp_case(activation)
    M, H = x.shape
    eps = r.eps64
    rs = 1.0 / np.sqrt(1.0 + eps)
    mf, mb = om.mlp_fwd_meta(r), om.mlp_bwd_meta(r)
    set_power_of_two_scales(mf, [1, 2, -1, 3])
    set_power_of_two_scales(mb, [2, 1])
    ones, zeros = exact_bf16(np.ones(H)), exact_bf16(np.zeros(H))
    out, ctx = om.ln_mlp_fwd(r, mf, exact_bf16(x), ones, zeros, exact_bf16(w1), exact_bf16(b1),
                             exact_bf16(w2), exact_bf16(b2))
    g = om.ln_mlp_bwd(r, mf, mb, exact_bf16(dy), ctx, exact_bf16(x), ones)

    w1_q, w2_q = rne(w1, ffmt), rne(w2, ffmt)
    h = x @ w1_q.T + b1                                # exact; GELU(h) = h here
    assert h.min() >= (8.0 if activation == oracle.GELU_TANH else 24.0)
    g_q = rne(h, ffmt)
    assert np.any(g_q != h), "the GELU output's cast must round somewhere"
    dy_q = rne(dy, bfmt)
    dh = dy_q @ w2_q                                   # GELU'(h) = 1
    dh_q = rne(dh, bfmt)
    assert np.any(dh_q != dh), "the fc1 gradient's cast must round somewhere"
    # forward
    np.testing.assert_array_equal(dec(ctx["ln_q"], ffmt, mf.scale_inv[0]), x)
    np.testing.assert_array_equal(oracle.bf16_to_f64(ctx["h_bits"]), h)
    np.testing.assert_array_equal(dec(ctx["g_q"], ffmt, mf.scale_inv[2]), g_q)
    np.testing.assert_array_equal(out, g_q @ w2_q.T + b2)
    assert mf.history[0, 0] == np.float32(rs)
    assert mf.history[0, 1] == np.float32(np.abs(w1).max())
    assert mf.history[0, 2] == np.float32(h.max())
    assert mf.history[0, 3] == np.float32(np.abs(w2).max())
    # backward
    np.testing.assert_array_equal(g["db2"], dy.sum(axis=0))
    np.testing.assert_array_equal(g["dh"], dh)
    np.testing.assert_array_equal(dec(g["dh_q"], bfmt, mb.scale_inv[1]), dh_q)
    np.testing.assert_array_equal(g["db1"], dh.sum(axis=0))
    np.testing.assert_array_equal(g["dw2"], dy_q.T @ g_q)
    dln = dh_q @ w1_q
    np.testing.assert_array_equal(g["dln"], dln)
    np.testing.assert_array_equal(g["dw1"], dh_q.T @ x)
    assert mb.history[0, 0] == np.float32(np.abs(dy).max())
    assert mb.history[0, 1] == np.float32(np.abs(dh).max())
    np.testing.assert_array_equal(g["dbeta"], dln.sum(axis=0))
    np.testing.assert_allclose(g["dgamma"], (dln * x).sum(axis=0) * rs, rtol=1e-14,
                               atol=1e-14 * np.abs(dln).sum(axis=0).max())
    np.testing.assert_allclose(g["dx"], ln_bwd_reference(dln, x, eps), rtol=1e-12,
                               atol=1e-12 * np.abs(dln).max())


@pytest.mark.parametrize("fmt", FORMATS)
def test_ln_mlp_chain_exact(fmt):
    check_ln_mlp_pins(oracle.modules, fmt)


@pytest.mark.parametrize("fmt", [oracle.FORMAT_HYBRID, oracle.FORMAT_E4M3])
def test_ln_mlp_chain_exact_erf(fmt):
    check_ln_mlp_pins(oracle.modules, fmt, oracle.GELU_ERF)


def test_gelu_is_identity_where_the_pins_use_it():
    """The pins rely on float64 GELU(h) = h and GELU'(h) = 1 from h = 8 (tanh
    form) and h = 24 (erf form) on: tanh(u) and erf rounds to 1 there."""
    h = np.arange(8.0, 40.0, 0.125)
    np.testing.assert_array_equal(oracle.gelu_tanh(h), h)
    np.testing.assert_array_equal(oracle.gelu_tanh_grad(h), np.ones_like(h))
    h = h[h >= 24.0]
    np.testing.assert_array_equal(oracle.gelu_erf(h), h)
    np.testing.assert_array_equal(oracle.gelu_erf_grad(h), np.ones_like(h))


def test_rne_helper_against_the_decode_table():
    """The pins' rounding helper agrees with the nearest FP8 value (ties to
    the even code) on a grid of normal-range values: it is the format's own
    rounding, written from the significand width."""
    for fmt in (E4M3, E5M2):
        pos = oracle.fp8_positive_values(fmt)
        pos = pos[pos >= MIN_NORMAL[fmt]]
        for lo, hi in zip(pos[:-1], pos[1:]):
            mid = (lo + hi) / 2
            assert rne(lo, fmt) == lo and rne(hi, fmt) == hi
            assert rne(np.nextafter(mid, 0), fmt) == lo
            assert rne(np.nextafter(mid, np.inf), fmt) == hi
            # the tie goes to the value whose last significand bit is 0
            m_lo = int(np.ldexp(lo, -(np.frexp(lo)[1] - 1 - MBITS[fmt])))
            assert rne(mid, fmt) == (lo if m_lo % 2 == 0 else hi)


# ---- mutations: each alternative reading must turn a pin red -------------------

def mutant(*subs):
    """A copy of oracle.modules with source substitutions (each must match
    exactly once), loaded as its own module."""
    src = inspect.getsource(oracle.modules)
    for old, new in subs:
        assert src.count(old) == 1, f"mutation site not found once: {old!r}"
        src = src.replace(old, new)
    name = "oracle._pin_mutant"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    mod.__file__ = oracle.modules.__file__
    sys.modules[name] = mod
    try:
        exec(compile(src, f"<mutant of {oracle.modules.__file__}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


_DEC = "__import__('oracle').fp8_decode"

MUTATIONS = {
    # wgrad of LayerNormLinear on the unquantised LN output instead of ln_q
    "ln_linear_wgrad_unquantised_ln": (
        "linear",
        ('dw = fp8_gemm_tn(dy_q.T, bfmt, ctx["ln_q"].T, ffmt, meta_bwd.scale_inv[0],\n'
         '                     meta_fwd.scale_inv[0])',
         f'dw = ({_DEC}(dy_q, bfmt).T @ ctx["y"]) * float(meta_bwd.scale_inv[0])')),
    # wgrad of Linear dequantised with the weight's scale_inv instead of the input's
    "linear_wgrad_wrong_scale": (
        "plain",
        ('dw = fp8_gemm_tn(dy_q.T, bfmt, ctx["x_q"].T, ffmt, meta_bwd.scale_inv[0],\n'
         '                     meta_fwd.scale_inv[0])',
         'dw = fp8_gemm_tn(dy_q.T, bfmt, ctx["x_q"].T, ffmt, meta_bwd.scale_inv[0],\n'
         '                     meta_fwd.scale_inv[1])')),
    # dbias from the quantised gradient
    "ln_linear_dbias_quantised": (
        "linear",
        ("    dbias = dy.sum(axis=0)\n",
         f"    dbias = ({_DEC}(dy_q, bfmt) * float(meta_bwd.scale_inv[0])).sum(axis=0)\n")),
    # dgrad dequantised with the LN output's scale_inv instead of the weight's
    "ln_linear_dgrad_wrong_scale": (
        "linear",
        ('dln = fp8_gemm_tn(dy_q, bfmt, ctx["w_q"].T, ffmt, meta_bwd.scale_inv[0], ctx["w_sinv"])',
         'dln = fp8_gemm_tn(dy_q, bfmt, ctx["w_q"].T, ffmt, meta_bwd.scale_inv[0], '
         'meta_fwd.scale_inv[0])')),
    # fc1 wgrad on the unquantised LN output
    "ln_mlp_wgrad1_unquantised_ln": (
        "mlp",
        ('dw1 = fp8_gemm_tn(dh_q.T, bfmt, ctx["ln_q"].T, ffmt, meta_bwd.scale_inv[1],\n'
         '                      meta_fwd.scale_inv[0])',
         f'dw1 = ({_DEC}(dh_q, bfmt).T @ ctx["y"]) * float(meta_bwd.scale_inv[1])')),
    # db1 from the quantised dH
    "ln_mlp_db1_quantised": (
        "mlp",
        ("db1 = dh.sum(axis=0)",
         f"db1 = ({_DEC}(dh_q, bfmt) * float(meta_bwd.scale_inv[1])).sum(axis=0)")),
    # fc2 wgrad on the unquantised GELU output instead of g_q
    "ln_mlp_wgrad2_unquantised_gelu": (
        "mlp",
        ('dw2 = fp8_gemm_tn(dy_q.T, bfmt, ctx["g_q"].T, ffmt, meta_bwd.scale_inv[0],\n'
         '                      meta_fwd.scale_inv[2])',
         f'dw2 = ({_DEC}(dy_q, bfmt).T @ ctx["g"]) * float(meta_bwd.scale_inv[0])')),
    # fc1 dgrad on the unquantised dH
    "ln_mlp_dgrad1_unquantised_dh": (
        "mlp",
        ('dln = fp8_gemm_tn(dh_q, bfmt, ctx["w1_q"].T, ffmt, meta_bwd.scale_inv[1], ctx["w1_sinv"])',
         f'dln = dh @ ({_DEC}(ctx["w1_q"], ffmt) * float(ctx["w1_sinv"]))')),
    # the GELU output cast with the fc2 weight's scale
    "ln_mlp_gelu_cast_wrong_slot": (
        "mlp",
        ("g_q, g_amax = cast_amax(g, meta.scale[2], fmt)",
         "g_q, g_amax = cast_amax(g, meta.scale[3], fmt)")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_reject_mutation(name):
    """Each planted alternative reading fails the exact pins (in every recipe
    where the two readings differ; at least in HYBRID)."""
    kind, sub = MUTATIONS[name]
    om = mutant(sub)
    check = {"linear": check_ln_linear_pins, "mlp": check_ln_mlp_pins,
             "plain": check_linear_pins}[kind]
    with pytest.raises(AssertionError):
        check(om, oracle.FORMAT_HYBRID)


def test_unmutated_copy_passes():
    """The mutation machinery itself: a copy with no change passes the pins."""
    om = mutant()
    check_ln_linear_pins(om, oracle.FORMAT_HYBRID)
    check_ln_mlp_pins(om, oracle.FORMAT_HYBRID)
