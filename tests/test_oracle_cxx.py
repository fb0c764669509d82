"""Pins for the C++ oracle (oracle/cpp/fp8ln_oracle.cpp, through oracle.cxx).

It is pinned on its own, not only against the Python oracle:

* the encoder over every binary32 input of both signs and both formats: in value
  order it is monotone and switches codes exactly at the midpoints of adjacent
  table values (ties to the even code), and NaN gives 0x7F; with the decode
  table's closed forms this makes it the brute-force nearest-value encoder on all
  2^32 inputs;
* the decode table against the OCP bit layouts' closed forms;
* the exact GEMM against rational brute force for all four format pairs
  (integer accumulation is exact where a float64 sum with E5M2 is only bounded);
* the scaling update's closed forms and a brute-force FIFO window;
* LayerNorm moments (gamma = 1, beta = 0: mean 0, variance var/(var + eps));
* the module chains through the same exact pins as the Python oracle
  (tests/test_oracle_module_pins.py), mutations included;

and then against the Python oracle on random inputs: codes, amaxes, scales and
histories bit for bit, float64 results to 1e-12.  A sanitizer build
(AddressSanitizer + UndefinedBehaviorSanitizer, host code only) runs the chains.
"""
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.cxx as X
from oracle import E4M3, E5M2

import test_oracle_module_pins as pins


@pytest.fixture(scope="module", autouse=True)
def built():
    X.lib()


# ---- codec --------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("negative", [False, True])
def test_encoder_on_every_binary32_input(fmt, negative):
    assert X.encode_check_sign(fmt, negative) == 0


def test_decode_table_closed_forms():
    e4, e5 = X.decode_table(E4M3), X.decode_table(E5M2)
    assert e4[0x7E] == 448.0 and np.isnan(e4[0x7F]) and np.isnan(e4[0xFF])
    assert e4[0x01] == 2.0 ** -9 and e4[0x08] == 2.0 ** -6 and e4[0x38] == 1.0
    assert e5[0x7B] == 57344.0 and e5[0x7C] == np.inf and e5[0xFC] == -np.inf
    assert all(np.isnan(e5[c]) for c in (0x7D, 0x7E, 0x7F))
    assert e5[0x01] == 2.0 ** -16 and e5[0x04] == 2.0 ** -14 and e5[0x3C] == 1.0
    for t, n in ((e4, 127), (e5, 124)):
        pos = t[:128][np.isfinite(t[:128])]
        assert len(pos) == n and np.all(np.diff(pos) > 0)
        np.testing.assert_array_equal(t[128:][np.isfinite(t[128:])], -pos)


def test_encoder_special_values():
    for fmt, mx in ((E4M3, 0x7E), (E5M2, 0x7B)):
        q = X.encode([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e300, -1e300], fmt)
        assert q.tolist() == [mx, mx | 0x80, 0x7F, 0x00, 0x80, mx, mx | 0x80]


def test_encoder_agrees_with_the_python_oracle_on_all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint16)
    v = oracle.bf16_to_f64(bits)
    for fmt in (E4M3, E5M2):
        for s in (1.0, 448.0 / 5.3, 2.0 ** -7, 57344.0 / 1e-3):
            np.testing.assert_array_equal(X.encode(v * s, fmt), oracle.fp8_encode(v * s, fmt))


def test_bf16_rounding_and_decoding():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(size=100000) * 10.0 ** rng.integers(-40, 40, 100000),
                        [0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-45]])
    np.testing.assert_array_equal(X.f64_to_bf16_bits(v), oracle.f64_to_bf16_bits(v))
    bits = np.arange(1 << 16, dtype=np.uint16)
    np.testing.assert_array_equal(X.bf16_to_f64(bits), oracle.bf16_to_f64(bits))


# ---- GEMM ---------------------------------------------------------------------

@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
def test_gemm_exact_against_rational_brute_force(fa, fb):
    """The integer accumulation gives the exact sum rounded once to float64 for
    every pair of formats, including full-range E5M2 operands whose float64
    sum would round."""
    M, N, K = 4, 5, 200
    rng = np.random.default_rng(7)
    ta, tb = oracle.fp8_decode_table(fa), oracle.fp8_decode_table(fb)
    fin_a = np.array([c for c in range(256) if np.isfinite(ta[c])], dtype=np.uint8)
    fin_b = np.array([c for c in range(256) if np.isfinite(tb[c])], dtype=np.uint8)
    a = rng.choice(fin_a, size=(M, K))
    b = rng.choice(fin_b, size=(N, K))
    c = X.fp8_gemm_tn(a, fa, b, fb)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(ta[a[i, k]])) * Fraction(float(tb[b[j, k]]))
                        for k in range(K))
            assert c[i, j] == float(exact)          # one correct rounding of the exact sum


def test_gemm_epilogue_and_layout():
    K = 48
    rng = np.random.default_rng(4)
    a = rng.integers(0, 0x7E, size=(6, K)).astype(np.uint8)
    perm = rng.permutation(K)
    b = np.zeros((K, K), dtype=np.uint8)
    b[np.arange(K), perm] = 0x38                 # 1.0: B selects columns of A
    bias = np.arange(K, dtype=np.float64)
    c = X.fp8_gemm_tn(a, E4M3, b, E4M3, np.float32(0.5), np.float32(4.0), bias)
    np.testing.assert_array_equal(c, oracle.fp8_decode(a, E4M3)[:, perm] * 2.0 + bias)


def test_gemm_matches_python_oracle_for_e4m3():
    rng = np.random.default_rng(5)
    a = rng.integers(0, 256, size=(33, 100)).astype(np.uint8)
    b = rng.integers(0, 256, size=(17, 100)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    b[(b & 0x7F) == 0x7F] = 0
    np.testing.assert_array_equal(X.fp8_gemm_tn(a, E4M3, b, E4M3, 0.25, 3.0),
                                  oracle.fp8_gemm_tn(a, E4M3, b, E4M3, 0.25, 3.0))


# ---- scaling --------------------------------------------------------------------

def _meta(L, fmts):
    return oracle.Meta.fresh(L, fmts)


def test_scaling_closed_forms():
    m = _meta(4, [E4M3, E4M3, E5M2, E4M3, E4M3, E4M3])
    m.history[2] = [448.0, 1.0, 57344.0, 0.0, np.inf, np.nan]
    X.scaling_update(m)
    assert m.scale.tolist()[:3] == [1.0, 448.0, 1.0]
    assert m.scale[3] == 1.0 and m.scale[4] == 1.0 and m.scale[5] == 1.0   # kept
    assert np.all(m.history[0] == 0) and m.history[3].tolist()[:3] == [448.0, 1.0, 57344.0]
    m2 = _meta(1, [E4M3])
    m2.history[0, 0] = 1.0
    X.scaling_update(m2, margin=1)
    assert m2.scale[0] == 224.0 and m2.scale_inv[0] == np.float32(1 / 224.0)
    m3 = _meta(1, [E4M3])
    m3.history[0, 0] = np.float32(1e-45)         # 448 / subnormal overflows binary32
    X.scaling_update(m3)
    assert m3.scale[0] == 1.0


def test_scaling_matches_python_oracle_and_the_fifo_window():
    rng = np.random.default_rng(9)
    for L in (1, 2, 16, 1024):
        mc, mp = _meta(L, [E4M3, E5M2, E4M3]), _meta(L, [E4M3, E5M2, E4M3])
        seen = []
        for step in range(40):
            X.scaling_update(mc)
            oracle.scaling_update(mp)
            vals = np.float32(rng.lognormal(size=3) * 10.0 ** rng.integers(-8, 8, size=3))
            if step % 13 == 5:
                vals[1] = np.nan
            for s in range(3):
                X.lib().orc_record_amax(mc.history.ctypes.data_as(X.C.c_void_p), s,
                                        float(vals[s]))
                mp.record_amax(s, vals[s])
            seen.append(vals)
            assert mc.history.tobytes() == mp.history.tobytes()
            assert mc.scale.tobytes() == mp.scale.tobytes()
            assert mc.scale_inv.tobytes() == mp.scale_inv.tobytes()
        # after an update the window max of the last L steps sets slot 0's scale
        X.scaling_update(mc)
        win = np.array(seen[-L:])[:, 0]
        assert mc.scale[0] == np.float32(448.0) / np.float32(win.max())


# ---- LayerNorm and GELU ---------------------------------------------------------

def test_layernorm_moments_and_python_oracle():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(64, 768)) * 3 + 1
    eps = float(np.float32(1e-5))
    y, mean, rstd = X.layernorm_fwd(x, np.ones(768), np.zeros(768), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-14)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)
    g, b = rng.normal(size=768), rng.normal(size=768)
    yc, mc, rc = X.layernorm_fwd(x, g, b, eps)
    yp, mp, rp = oracle.layernorm_fwd(x, g, b, eps)
    np.testing.assert_allclose(yc, yp, rtol=1e-13, atol=1e-13)
    dy = rng.normal(size=x.shape)
    for c, p in zip(X.layernorm_bwd(dy, x, g, mc, rc), oracle.layernorm_bwd(dy, x, g, mp, rp)):
        np.testing.assert_allclose(c, p, rtol=1e-11, atol=1e-12)


def test_gelu_matches_python_oracle():
    """Same formulas, two libm's: equal to a few ulps of the inputs' scale (the
    tanh and erf forms cancel for negative h, so small results carry an
    absolute, not relative, error of that size in both)."""
    h = np.linspace(-12, 12, 20001)
    for act, f, fg in ((X.GELU_TANH, oracle.gelu_tanh, oracle.gelu_tanh_grad),
                       (X.GELU_ERF, oracle.gelu_erf, oracle.gelu_erf_grad)):
        np.testing.assert_allclose(X.gelu(h, act), f(h), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(X.gelu_grad(h, act), fg(h), rtol=1e-13, atol=1e-14)


# ---- module chains: the exact pins, then the Python oracle ----------------------

@pytest.mark.parametrize("fmt", pins.FORMATS)
def test_cxx_ln_linear_exact_pins(fmt):
    pins.check_ln_linear_pins(X, fmt)


@pytest.mark.parametrize("fmt", pins.FORMATS)
def test_cxx_ln_mlp_exact_pins(fmt):
    pins.check_ln_mlp_pins(X, fmt)


def test_cxx_ln_mlp_exact_pins_erf():
    pins.check_ln_mlp_pins(X, oracle.FORMAT_HYBRID, oracle.GELU_ERF)


def _lin_case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    b = oracle.f64_to_bf16_bits
    return (b(rng.normal(size=(M, K))), b(1 + 0.1 * rng.normal(size=K)),
            b(0.1 * rng.normal(size=K)), b(0.02 * rng.normal(size=(N, K))),
            b(0.1 * rng.normal(size=N)), b(1e-3 * rng.normal(size=(M, N))))


def _ln_codes_agree(qc, qp, y, scale, fmt):
    """LN codes: equal, except where the two float64 LayerNorms (summed in
    different orders) fall on either side of a rounding midpoint."""
    diff = qc != qp
    if diff.any():
        v = y[diff] * float(scale)
        lo = oracle.fp8_encode(v * (1 - 1e-13), fmt)
        hi = oracle.fp8_encode(v * (1 + 1e-13), fmt)
        assert np.all(lo != hi), "LN code differs away from a rounding midpoint"
    return int(diff.sum())


@pytest.mark.parametrize("fmt", [oracle.FORMAT_HYBRID, oracle.FORMAT_E4M3])
def test_cxx_ln_linear_chain_matches_python_oracle(fmt):
    r = oracle.Recipe(format=fmt)
    mfc, mbc = oracle.linear_fwd_meta(r), oracle.linear_bwd_meta(r)
    mfp, mbp = oracle.linear_fwd_meta(r), oracle.linear_bwd_meta(r)
    for step in range(4):
        x, g, b, w, bias, dy = _lin_case(96, 128, 80, step)
        for m in (mfc, mbc):
            X.scaling_update(m)
        for m in (mfp, mbp):
            oracle.scaling_update(m)
        oc, cc = X.ln_linear_fwd(r, mfc, x, g, b, w, bias)
        op, cp = oracle.ln_linear_fwd(r, mfp, x, g, b, w, bias)
        gc = X.ln_linear_bwd(r, mfc, mbc, dy, cc, x, g)
        gp = oracle.ln_linear_bwd(r, mfp, mbp, dy, cp, x, g)
        _ln_codes_agree(cc["ln_q"], cp["ln_q"], cp["y"], mfp.scale[0], oracle.fwd_format(r))
        np.testing.assert_array_equal(cc["w_q"], cp["w_q"])
        np.testing.assert_array_equal(gc["dy_q"], gp["dy_q"])
        for m1, m2 in ((mfc, mfp), (mbc, mbp)):
            assert np.allclose(m1.history, m2.history, rtol=1e-7, atol=0)
            assert m1.scale.tobytes() == m2.scale.tobytes()
        if not np.array_equal(cc["ln_q"], cp["ln_q"]):
            continue    # a flipped LN code moves the products below; skip exactness
        np.testing.assert_allclose(oc, op, rtol=1e-12, atol=1e-12)
        for k in ("dx", "dgamma", "dbeta", "dw", "dbias", "dln"):
            np.testing.assert_allclose(gc[k], gp[k], rtol=1e-11, atol=1e-15, err_msg=k)


@pytest.mark.parametrize("fmt,act", [(oracle.FORMAT_HYBRID, oracle.GELU_TANH),
                                     (oracle.FORMAT_E4M3, oracle.GELU_ERF)])
def test_cxx_ln_mlp_chain_matches_python_oracle(fmt, act):
    r = oracle.Recipe(format=fmt, activation=act)
    mfc, mbc = oracle.mlp_fwd_meta(r), oracle.mlp_bwd_meta(r)
    mfp, mbp = oracle.mlp_fwd_meta(r), oracle.mlp_bwd_meta(r)
    rng = np.random.default_rng(21)
    bits = oracle.f64_to_bf16_bits
    M, H, F = 64, 64, 192
    for step in range(3):
        x = bits(rng.normal(size=(M, H)))
        g, b = bits(1 + 0.1 * rng.normal(size=H)), bits(0.1 * rng.normal(size=H))
        w1, w2 = bits(0.1 * rng.normal(size=(F, H))), bits(0.1 * rng.normal(size=(H, F)))
        b1, b2 = bits(0.1 * rng.normal(size=F)), bits(0.1 * rng.normal(size=H))
        dy = bits(1e-3 * rng.normal(size=(M, H)))
        for m in (mfc, mbc):
            X.scaling_update(m)
        for m in (mfp, mbp):
            oracle.scaling_update(m)
        oc, cc = X.ln_mlp_fwd(r, mfc, x, g, b, w1, b1, w2, b2)
        op, cp = oracle.ln_mlp_fwd(r, mfp, x, g, b, w1, b1, w2, b2)
        gc = X.ln_mlp_bwd(r, mfc, mbc, dy, cc, x, g)
        gp = oracle.ln_mlp_bwd(r, mfp, mbp, dy, cp, x, g)
        np.testing.assert_array_equal(cc["w1_q"], cp["w1_q"])
        np.testing.assert_array_equal(cc["w2_q"], cp["w2_q"])
        np.testing.assert_array_equal(gc["dy_q"], gp["dy_q"])
        assert np.array_equal(cc["ln_q"], cp["ln_q"]), "no LN code near a midpoint here"
        np.testing.assert_allclose(cc["h"], cp["h"], rtol=1e-13, atol=1e-14)
        assert np.array_equal(cc["h_bits"], cp["h_bits"])
        assert np.array_equal(cc["g_q"], cp["g_q"])
        assert np.array_equal(gc["dh_q"], gp["dh_q"])
        for m1, m2 in ((mfc, mfp), (mbc, mbp)):
            np.testing.assert_allclose(m1.history, m2.history, rtol=1e-7)
            assert m1.scale.tobytes() == m2.scale.tobytes()
        np.testing.assert_allclose(oc, op, rtol=1e-12, atol=1e-13)
        for k in ("dx", "dgamma", "dbeta", "dw1", "db1", "dw2", "db2", "dh", "dln"):
            np.testing.assert_allclose(gc[k], gp[k], rtol=1e-10, atol=1e-16, err_msg=k)


def test_cxx_standalone_ln_cast_amax_matches_chain_step():
    rng = np.random.default_rng(2)
    bits = oracle.f64_to_bf16_bits
    x = bits(rng.normal(size=(256, 1024)) * 2)
    g, b = bits(1 + 0.1 * rng.normal(size=1024)), bits(0.1 * rng.normal(size=1024))
    eps = float(np.float32(1e-5))
    q, a, mean, rstd = X.ln_cast_amax(x, g, b, eps, np.float32(60.0), E4M3)
    y, mp, rp = oracle.layernorm_fwd(oracle.bf16_to_f64(x), oracle.bf16_to_f64(g),
                                     oracle.bf16_to_f64(b), eps)
    _ln_codes_agree(q, oracle.fp8_encode(y * float(np.float32(60.0)), E4M3), y, 60.0, E4M3)
    assert a == np.float32(np.abs(y).max())
    # sequential against pairwise float64 sums over 1024 entries
    np.testing.assert_allclose(mean, mp, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(rstd, rp, rtol=1e-13)


# ---- sanitizer build ---------------------------------------------------------------

SELFTEST = os.path.join(os.path.dirname(X.SRC), "selftest.cpp")


def test_sanitizer_build_runs_clean(tmp_path):
    """The oracle's chains under AddressSanitizer and UndefinedBehaviorSanitizer
    (host code, g++): no invalid access, leak or undefined operation."""
    exe = str(tmp_path / "oracle_selftest")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", exe, SELFTEST]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "selftest ok" in r.stdout
