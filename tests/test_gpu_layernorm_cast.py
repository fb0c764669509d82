"""GPU parity: fused LayerNorm + FP8 cast + amax, the tensor cast (weights and
gradients, with transposes and column sums) and the LayerNorm backward."""
import numpy as np
import pytest
import torch

import oracle
from fp8_delayed_scaling_row_amd import inputs, ops
from parity import (assert_vector_close, compare_bf16, compare_codes, ln_window, to_np,
                    to_np_bits)

pytestmark = pytest.mark.gpu

FMT = {ops.E4M3: oracle.E4M3, ops.E5M2: oracle.E5M2}


def _scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _oracle_ln(x_bits, g_bits, b_bits, eps, scale, fmt):
    x = oracle.bf16_to_f64(x_bits)
    g = oracle.bf16_to_f64(g_bits)
    b = oracle.bf16_to_f64(b_bits)
    y, mean, rstd = oracle.layernorm_fwd(x, g, b, eps)
    gx = (x - mean[:, None]) * rstd[:, None] * g
    return y, mean, rstd, gx, b


@pytest.mark.parametrize("rows,hidden,fp8,with_t,scale", [
    (1, 8, ops.E4M3, False, 1.0),
    (37, 768, ops.E4M3, False, 448.0 / 5.3),
    (256, 768, ops.E4M3, True, 448.0 / 5.3),
    (300, 2048, ops.E4M3, False, 74.0),
    (48, 1024, ops.E5M2, True, 5000.0),
    (64, 8192, ops.E4M3, False, 60.0),
    (16, 4096, ops.E4M3, True, 1.0),
    (272, 208, ops.E5M2, True, 300.0),   # transposed tiles cut on both edges
    (0, 768, ops.E4M3, False, 1.0),
])
def test_ln_cast_amax_matches_oracle(rows, hidden, fp8, with_t, scale):
    wl = f"ln/{rows}x{hidden}"
    x = inputs.spiky_normal_bf16((rows, hidden), inputs.seed_for(wl, "x"), drift=1.5)
    g, b = inputs.layernorm_params(hidden, wl)
    xd, gd, bd = x.cuda(), g.cuda(), b.cuda()
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    out_t = torch.empty((hidden, rows), dtype=torch.uint8, device="cuda") if with_t else None
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    r = ops.Recipe()
    ops.ln_cast_amax(r, xd, gd, bd, fp8, _scalar(scale), amax.data_ptr(), out, out_t, mean, rstd)
    torch.cuda.synchronize()
    if rows == 0:
        assert amax.item() == 0.0
        return
    fmt = FMT[fp8]
    y, om, orstd, gx, beta = _oracle_ln(to_np_bits(x), to_np_bits(g), to_np_bits(b),
                                         float(np.float32(r.ln_eps)), scale, fmt)
    sc = float(np.float32(scale))
    exact = y * sc
    stats = compare_codes(out.cpu().numpy(), exact, fmt, ln_window(gx, beta, sc, exact))
    oamax = np.float32(np.abs(y).max())
    assert abs(float(amax.item()) - float(oamax)) <= 1e-6 * float(oamax), (amax.item(), oamax)
    np.testing.assert_allclose(mean.cpu().numpy(), om, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(rstd.cpu().numpy(), orstd, rtol=1e-5)
    if with_t:
        assert torch.equal(out_t, out.t().contiguous())
    print(f"ln_cast_amax {rows}x{hidden}: {stats}")


def test_ln_cast_amax_nan_and_inf_rows():
    rows, hidden = 32, 256
    x = inputs.normal_bf16((rows, hidden), inputs.seed_for("ln-nan", "x"))
    x[3, 17] = float("nan")
    x[9, 0] = float("inf")
    g, b = inputs.layernorm_params(hidden, "ln-nan")
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.ln_cast_amax(ops.Recipe(), x.cuda(), g.cuda(), b.cuda(), ops.E4M3, _scalar(2.0),
                     amax.data_ptr(), out)
    torch.cuda.synchronize()
    q = out.cpu().numpy()
    assert np.all(q[3] == 0x7F) and np.all(q[9] == 0x7F)   # whole rows become NaN
    assert np.isnan(amax.item())
    y, *_ = _oracle_ln(to_np_bits(x), to_np_bits(g), to_np_bits(b), float(np.float32(1e-5)),
                       2.0, oracle.E4M3)
    ok = np.ones(rows, bool)
    ok[[3, 9]] = False
    np.testing.assert_array_equal(q[~ok], oracle.fp8_encode(y[~ok] * 2.0, oracle.E4M3))


def test_ln_cast_amax_full_size_sampled():
    """65536 x 2048 with 0.1 % spikes and drift 4: every row's amax, and the
    codes of 512 sampled rows plus the first and last rows."""
    rows, hidden = 65536, 2048
    x = inputs.spiky_normal_bf16((rows, hidden), inputs.seed_for("ln-full", "x"), drift=4.0,
                                 device="cuda")
    g, b = inputs.layernorm_params(hidden, "ln-full", device="cuda")
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    scale = 448.0 / 60.0
    ops.ln_cast_amax(ops.Recipe(amax_history_len=1024, format=ops.FORMAT_E4M3), x, g, b,
                     ops.E4M3, _scalar(scale), amax.data_ptr(), out)
    torch.cuda.synchronize()
    xb, gb, bb = to_np_bits(x), to_np_bits(g), to_np_bits(b)
    eps = float(np.float32(1e-5))
    oamax = 0.0
    for r0 in range(0, rows, 8192):
        y, *_ = _oracle_ln(xb[r0:r0 + 8192], gb, bb, eps, scale, oracle.E4M3)
        oamax = max(oamax, float(np.abs(y).max()))
    oamax = float(np.float32(oamax))
    assert abs(amax.item() - oamax) <= 1e-6 * oamax
    sample = np.unique(np.concatenate([[0, rows - 1],
                                       np.random.default_rng(1).integers(0, rows, 512)]))
    y, _, _, gx, beta = _oracle_ln(xb[sample], gb, bb, eps, scale, oracle.E4M3)
    sc = float(np.float32(scale))
    q = out[torch.from_numpy(sample).cuda()].cpu().numpy()
    stats = compare_codes(q, y * sc, oracle.E4M3, ln_window(gx, beta, sc, y * sc))
    print(f"full-size sample: {stats}")


@pytest.mark.parametrize("rows,cols,in_f32,fp8,with_t,with_sum,scale_from", [
    (16, 16, False, ops.E4M3, True, True, None),
    (2304, 768, False, ops.E4M3, True, False, None),
    (2048, 2304, False, ops.E5M2, True, True, None),
    (48, 80, False, ops.E4M3, True, True, None),
    (100, 48, True, ops.E5M2, False, True, None),
    (256, 3072, True, ops.E5M2, True, True, None),
    (0, 64, False, ops.E4M3, False, True, None),
    (2048, 2304, False, ops.E5M2, True, True, "amax"),
    (2304, 768, False, ops.E4M3, True, False, "amax"),
])
def test_cast_amax_matches_oracle(rows, cols, in_f32, fp8, with_t, with_sum, scale_from):
    """scale_from="amax": the scale a delayed-scaling step would use,
    fp8_max / amax of the same bf16 data; its products with the data hit FP8
    rounding midpoints after a binary32 rounding for whole mantissa patterns."""
    wl = f"cast/{rows}x{cols}"
    if in_f32:
        xf = torch.randn((rows, cols), generator=torch.Generator().manual_seed(5)) * 3e-4
        x = xf.to(torch.float32)
        xv = x.numpy().astype(np.float64)
    else:
        x = inputs.normal_bf16((rows, cols), inputs.seed_for(wl, "x"), std=0.02)
        xv = oracle.bf16_to_f64(to_np_bits(x))
    xd = x.cuda()
    out = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    out_t = torch.empty((cols, rows), dtype=torch.uint8, device="cuda") if with_t else None
    colsum = torch.full((cols,), 7.0, dtype=torch.float32, device="cuda") if with_sum else None
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    scale = float(np.float32(448.0 / 0.093 if fp8 == ops.E4M3 else 57344.0 / 0.0011))
    if scale_from == "amax" and rows:
        fmax = np.float32(448.0 if fp8 == ops.E4M3 else 57344.0)
        scale = float(fmax / np.float32(np.abs(xv).max()))
    ops.cast_amax(xd, fp8, _scalar(scale), amax.data_ptr(), out, out_t, colsum)
    torch.cuda.synchronize()
    if with_sum:
        ref = xv.sum(axis=0)
        got = colsum.cpu().numpy()
        bound = 1e-5 * np.abs(xv).sum(axis=0) + 1e-30
        assert np.all(np.abs(got - ref) <= bound), np.abs(got - ref).max()
    if rows == 0:
        assert amax.item() == 0.0
        return
    fmt = FMT[fp8]
    exact = xv * scale
    # the cast scales with a round-to-odd product: codes equal the oracle's
    stats = compare_codes(out.cpu().numpy(), exact, fmt, 0.0)
    assert stats["mismatched"] == 0
    assert np.float32(amax.item()) == np.float32(np.abs(xv).max())     # exact for these inputs
    if with_t:
        assert torch.equal(out_t, out.t().contiguous())
    print(f"cast {rows}x{cols}: {stats}")


@pytest.mark.parametrize("fp8", [ops.E4M3, ops.E5M2])
@pytest.mark.parametrize("in_f32", [False, True])
@pytest.mark.parametrize("with_nan", [False, True])
def test_cast_amax_infinities_nan_and_overflow(fp8, in_f32, with_nan):
    """Weights and gradients may hold infinities, NaNs or values whose scaled
    product overflows binary32: infinities and overflowing products saturate to
    +-max, NaN encodes to 0x7F, and the amax is inf (NaN when a NaN is
    present), all as the oracle encodes the exact products."""
    rows, cols = 96, 160
    rng = np.random.default_rng(11 + 2 * fp8 + int(in_f32))
    xv = rng.normal(size=(rows, cols)) * 0.02
    flat = xv.reshape(-1)
    idx = rng.permutation(flat.size)
    flat[idx[0:7]] = np.inf
    flat[idx[7:14]] = -np.inf
    flat[idx[14:30]] = 3.0e38 * rng.choice([-1.0, 1.0], size=16)    # product overflows
    flat[idx[30:60]] = rng.normal(size=30) * 1e4                     # past +-max after scaling
    if with_nan:
        flat[idx[60:63]] = np.nan
    if in_f32:
        x = torch.from_numpy(xv.astype(np.float32))
        xv = x.numpy().astype(np.float64)
    else:
        bits = oracle.f64_to_bf16_bits(xv)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        xv = oracle.bf16_to_f64(bits)
    out = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    out_t = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    scale = float(np.float32(448.0 / 0.093 if fp8 == ops.E4M3 else 57344.0 / 0.0011))
    ops.cast_amax(x.cuda(), fp8, _scalar(scale), amax.data_ptr(), out, out_t, None)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        exact = xv * scale
    stats = compare_codes(out.cpu().numpy(), exact, FMT[fp8], 0.0)
    assert stats["mismatched"] == 0
    assert torch.equal(out_t, out.t().contiguous())
    a = amax.item()
    assert np.isnan(a) if with_nan else a == np.inf


# hidden 1544 and 3080: the last chunk of a lane is past the row for all lanes but
# one (four chunks per lane) or for most (eight per lane), so the masking of the
# chunks past the row is exercised at every per-lane chunk count
@pytest.mark.parametrize("rows,hidden", [(1, 8), (37, 768), (2048, 768), (513, 2048),
                                         (64, 4096), (0, 256), (130, 1544), (70, 3080)])
def test_layernorm_bwd_matches_oracle(rows, hidden):
    wl = f"lnb/{rows}x{hidden}"
    x = inputs.normal_bf16((rows, hidden), inputs.seed_for(wl, "x"))
    g, b = inputs.layernorm_params(hidden, wl)
    dy = inputs.normal_bf16((rows, hidden), inputs.seed_for(wl, "dy"), std=1e-3).float()
    xv = oracle.bf16_to_f64(to_np_bits(x))
    gv = oracle.bf16_to_f64(to_np_bits(g))
    _, mean, rstd = oracle.layernorm_fwd(xv, gv, oracle.bf16_to_f64(to_np_bits(b)),
                                         float(np.float32(1e-5)))
    mean32, rstd32 = mean.astype(np.float32), rstd.astype(np.float32)
    dx = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    dgamma = torch.empty(hidden, dtype=torch.float32, device="cuda")
    dbeta = torch.empty(hidden, dtype=torch.float32, device="cuda")
    ops.layernorm_bwd(dy.cuda(), x.cuda(), torch.from_numpy(mean32).cuda(),
                      torch.from_numpy(rstd32).cuda(), g.cuda(), dx, dgamma, dbeta)
    torch.cuda.synchronize()
    odx, odg, odb = oracle.layernorm_bwd(dy.numpy().astype(np.float64), xv, gv,
                                         mean32.astype(np.float64), rstd32.astype(np.float64))
    if rows == 0:
        assert torch.all(dgamma == 0) and torch.all(dbeta == 0)
        return
    gdx = to_np(dx)
    norms = np.linalg.norm(odx, axis=1)
    assert np.all(np.abs(gdx - odx).max(axis=1) <= 1e-2 * norms + 1e-30)   # bf16 output
    assert_vector_close(dgamma.cpu().numpy(), odg, 1e-5, "dgamma")
    assert_vector_close(dbeta.cpu().numpy(), odb, 1e-5, "dbeta")


# ---- the plain LayerNorm module -------------------------------------------------

@pytest.mark.parametrize("rows,hidden", [(1, 8), (37, 768), (256, 768), (300, 2048),
                                         (64, 8192), (2000, 1000), (0, 768)])
def test_layernorm_module_fwd_matches_oracle(rows, hidden):
    """bf16 LayerNorm output: the rounding of the float64 result, or its
    neighbour where the fp32 result lies within the LayerNorm window of a bf16
    rounding midpoint; mean and rstd as in the fused LayerNorm's test."""
    wl = f"lnm/{rows}x{hidden}"
    x = inputs.normal_bf16((rows, hidden), inputs.seed_for(wl, "x"), std=3.0, mean=1.0)
    g, b = inputs.layernorm_params(hidden, wl)
    y = torch.full((rows, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    ops.layernorm_fwd(x.cuda(), g.cuda(), b.cuda(), y, mean, rstd)
    torch.cuda.synchronize()
    eps = float(np.float32(1e-5))
    ref = oracle.layernorm(to_np_bits(x), to_np_bits(g), to_np_bits(b), eps)
    if rows == 0:
        return
    # Rows here have a non-zero mean, so x - mean cancels: an fp32 mean carries an
    # absolute error that is small against |x| + |mean| but not against |x - mean|.
    # The window is 1e-6 of the magnitudes entering the computation:
    # |gamma| rstd (|x| + |mean|) + |beta|, and |y| itself.
    xv = oracle.bf16_to_f64(to_np_bits(x))
    gv, bv = (oracle.bf16_to_f64(to_np_bits(t)) for t in (g, b))
    mag = np.abs(gv) * ref["rstd"][:, None] * (np.abs(xv) + np.abs(ref["mean"])[:, None]) + \
        np.abs(bv)
    stats = compare_bf16(to_np_bits(y), ref["y"], 1e-6 * np.maximum(np.abs(ref["y"]), mag))
    np.testing.assert_allclose(mean.cpu().numpy(), ref["mean"], rtol=1e-5,
                               atol=1e-6 * np.abs(oracle.bf16_to_f64(to_np_bits(x))).max())
    np.testing.assert_allclose(rstd.cpu().numpy(), ref["rstd"], rtol=1e-5)
    assert stats["mismatched"] <= 2 + stats["n"] // 200, stats
    print(f"layernorm {rows}x{hidden}: {stats}")


# hidden 1544 and 3080: the last chunk of a lane is past the row for all lanes but
# one (four chunks per lane) or for most (eight per lane), so the masking of the
# chunks past the row is exercised at every per-lane chunk count
@pytest.mark.parametrize("rows,hidden", [(1, 8), (37, 768), (2048, 768), (513, 2048),
                                         (64, 4096), (0, 256), (130, 1544), (70, 3080)])
def test_layernorm_module_bwd_bf16_grad(rows, hidden):
    """The plain LayerNorm backward with a bf16 incoming gradient against the
    oracle's float64 backward; and on the same values it equals the fp32-gradient
    entry bit for bit."""
    wl = f"lnmb/{rows}x{hidden}"
    x = inputs.normal_bf16((rows, hidden), inputs.seed_for(wl, "x"))
    g, b = inputs.layernorm_params(hidden, wl)
    dy = inputs.normal_bf16((rows, hidden), inputs.seed_for(wl, "dy"), std=1e-2)
    xd, gd, bd = x.cuda(), g.cuda(), b.cuda()
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    y = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
    ops.layernorm_fwd(xd, gd, bd, y, mean, rstd)
    outs = []
    for dyd in (dy.cuda(), dy.float().cuda()):
        dx = torch.empty((rows, hidden), dtype=torch.bfloat16, device="cuda")
        dgamma = torch.empty(hidden, dtype=torch.float32, device="cuda")
        dbeta = torch.empty(hidden, dtype=torch.float32, device="cuda")
        if dyd.dtype == torch.bfloat16:
            ops.layernorm_bwd_bf16(dyd, xd, mean, rstd, gd, dx, dgamma, dbeta)
        else:
            ops.layernorm_bwd(dyd, xd, mean, rstd, gd, dx, dgamma, dbeta)
        outs.append((dx, dgamma, dbeta))
    torch.cuda.synchronize()
    for a, c in zip(*outs):
        assert torch.equal(a, c)
    dx, dgamma, dbeta = outs[0]
    if rows == 0:
        assert torch.all(dgamma == 0) and torch.all(dbeta == 0)
        return
    m64, r64 = mean.cpu().numpy().astype(np.float64), rstd.cpu().numpy().astype(np.float64)
    xv, gv = oracle.bf16_to_f64(to_np_bits(x)), oracle.bf16_to_f64(to_np_bits(g))
    odx, odg, odb = oracle.layernorm_bwd(oracle.bf16_to_f64(to_np_bits(dy)), xv, gv, m64, r64)
    gdx = to_np(dx)
    norms = np.linalg.norm(odx, axis=1)
    assert np.all(np.abs(gdx - odx).max(axis=1) <= 1e-2 * norms + 1e-30)   # bf16 output
    assert_vector_close(dgamma.cpu().numpy(), odg, 1e-5, "dgamma")
    assert_vector_close(dbeta.cpu().numpy(), odb, 1e-5, "dbeta")


def test_ln_cast_amax_32_drifting_steps_history_1024():
    """The LN + cast + amax workload over its 32 steps: 65536 x 2048 rows of
    N(0,1) with 0.1 % of entries x100 and the input scale drifting 1 -> 4, E4M3,
    history 1024.  Every step: the scale update's history, scale and scale_inv
    bit-exact against the oracle's (fed the GPU's recorded amaxes, identical-input
    mode), the step's LayerNorm-output amax within 1e-6 relative of the oracle's
    over all rows (C++ oracle, float64), and the codes of sampled rows by the
    LayerNorm code rule."""
    import oracle.cxx as X
    rows, hidden, steps = 65536, 2048, 32
    recipe = ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=1024)
    meta = ops.Meta(recipe, 1, ops.META_FORWARD)
    om = oracle.Meta.fresh(1024, [oracle.E4M3])
    wl = "ln_cast_amax_65536x2048"
    g, b = inputs.layernorm_params(hidden, wl)
    gd, bd = g.cuda(), b.cuda()
    gb, bb = to_np_bits(g), to_np_bits(b)
    eps = float(np.float32(1e-5))
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(32)
    for s in range(steps):
        print(f"c1 step {s}", flush=True)
        x = inputs.spiky_normal_bf16((rows, hidden), inputs.seed_for(wl, "x", s),
                                     drift=inputs.drift_factor(s, steps), device="cuda")
        ops.scaling_update(recipe, meta)
        oracle.scaling_update(om)
        torch.cuda.synchronize()
        for name in ("history", "scale", "scale_inv"):
            got = getattr(meta, name).cpu().numpy().reshape(-1).view(np.uint32)
            want = getattr(om, name).reshape(-1).view(np.uint32)
            assert np.array_equal(got, want), f"step {s}: {name} differs"
        ops.ln_cast_amax(recipe, x, gd, bd, ops.E4M3, meta.scale[0:1], meta.amax_ptr(0), out)
        torch.cuda.synchronize()
        gpu_amax = np.float32(meta.history[0, 0].item())
        xb = to_np_bits(x)
        sc = np.float32(om.scale[0])
        _, oamax, _, _ = X.ln_cast_amax(xb, gb, bb, eps, sc, oracle.E4M3, stats=False)
        assert abs(float(gpu_amax) - float(oamax)) <= 1e-6 * float(oamax), (s, gpu_amax, oamax)
        om.record_amax(0, gpu_amax)          # identical input for the next update
        sample = rng.integers(0, rows, 48)
        y, _, _, gx, beta = _oracle_ln(xb[sample], gb, bb, eps, sc, oracle.E4M3)
        compare_codes(out[torch.from_numpy(sample).cuda()].cpu().numpy(), y * float(sc),
                      oracle.E4M3, ln_window(gx, beta, float(sc), y * float(sc)))
    assert np.float32(meta.scale[0].item()) != 1.0
