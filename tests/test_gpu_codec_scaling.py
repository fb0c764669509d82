"""GPU parity: the device FP8 encoder on every binary32 input, and the
delayed-scaling state update, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from fp8_delayed_scaling_row_amd import inputs, ops

pytestmark = pytest.mark.gpu

FMT = {ops.E4M3: oracle.E4M3, ops.E5M2: oracle.E5M2}


def oracle_runs(fmt: str):
    """Runs of the oracle encoder over all 2^32 binary32 patterns, as sorted
    (first pattern, code) pairs.  Over the non-negative patterns 0 .. 0x7f800000
    the encoder is non-decreasing (pinned on the CPU), so each code's first
    pattern is found by bisection with the oracle itself."""
    maxc = len(oracle.fp8_positive_values(fmt)) - 1

    def enc(bits):
        b = np.asarray(bits, dtype=np.uint32)
        return oracle.fp8_encode(b.view(np.float32).astype(np.float64), fmt).astype(np.int64)

    codes = np.arange(1, maxc + 1)
    lo = np.zeros(maxc, dtype=np.int64)               # enc(lo) < code
    hi = np.full(maxc, 0x7F800000, dtype=np.int64)    # enc(hi) >= code (+inf saturates)
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        ge = enc(mid) >= codes
        hi = np.where(ge, mid, hi)
        lo = np.where(ge, lo, mid)
    runs = [(0, 0x00)] + [(int(h), int(c)) for h, c in zip(hi, codes)]
    runs += [(0x7F800001, 0x7F), (0x80000000, 0x80)]
    runs += [(0x80000000 + int(h), 0x80 | int(c)) for h, c in zip(hi, codes)]
    runs += [(0xFF800001, 0x7F)]
    return runs


@pytest.mark.parametrize("fp8", [ops.E4M3, ops.E5M2], ids=["e4m3", "e5m2"])
def test_encoder_equals_cxx_oracle_on_every_float32(fp8):
    """Element by element over all 2^32 binary32 patterns against the C++
    oracle's table-exact encoder (which is itself checked exhaustively against
    the nearest-value definition on the CPU)."""
    import oracle.cxx as X
    fmt = FMT[fp8]
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    ref = np.empty(chunk, dtype=np.uint8)
    for base in range(0, 1 << 32, chunk):
        ops.encode_range(base, chunk, fp8, out)
        X.encode_f32_range(base, chunk, fmt, ref)
        got = out.cpu().numpy()
        if not np.array_equal(got, ref):
            i = int(np.nonzero(got != ref)[0][0])
            raise AssertionError(f"pattern {base + i:#x}: gpu {got[i]:#x} oracle {ref[i]:#x}")


def test_stream_probe_picks_the_high_bytes():
    x = inputs.normal_bf16(((1 << 20) + 8,), inputs.seed_for("probe", "x"), device="cuda")
    out = torch.empty(x.numel(), dtype=torch.uint8, device="cuda")
    ops.stream_probe(x, out)
    want = (x.view(torch.int16).to(torch.int32) >> 8) & 0xFF
    assert torch.equal(out.to(torch.int32), want)


@pytest.mark.parametrize("fp8", [ops.E4M3, ops.E5M2], ids=["e4m3", "e5m2"])
def test_encoder_matches_oracle_on_every_float32(fp8):
    fmt = FMT[fp8]
    runs = oracle_runs(fmt)
    starts = np.array([r[0] for r in runs], dtype=np.int64)
    vals = np.array([r[1] for r in runs], dtype=np.int64)
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    for base in range(0, 1 << 32, chunk):
        ops.encode_range(base, chunk, fp8, out)
        d = torch.nonzero(out[1:] != out[:-1]).flatten() + 1
        pos = d.cpu().numpy().astype(np.int64)
        got_vals = out[d].cpu().numpy().astype(np.int64)
        first = int(out[0].item())
        # expected: code at `base` and every run start inside (base, base + chunk)
        k = np.searchsorted(starts, base, side="right") - 1
        assert first == vals[k], f"pattern {base:#x}: gpu {first:#x} oracle {vals[k]:#x}"
        inside = (starts > base) & (starts < base + chunk)
        np.testing.assert_array_equal(pos, starts[inside] - base,
                                      err_msg=f"run starts differ in chunk {base:#x}")
        np.testing.assert_array_equal(got_vals, vals[inside])


def _fmt_of(recipe, kind):
    if recipe.format == ops.FORMAT_E4M3:
        return oracle.E4M3
    if recipe.format == ops.FORMAT_E5M2:
        return oracle.E5M2
    return oracle.E4M3 if kind == 0 else oracle.E5M2


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def test_meta_init_state():
    r = ops.Recipe(amax_history_len=16)
    m = ops.Meta(r, 4, 0, init=False)
    m.history.fill_(7.0)
    m.scale.fill_(3.0)
    m.scale_inv.fill_(5.0)
    ops.meta_init(r, m)
    torch.cuda.synchronize()
    assert torch.all(m.history == 0) and torch.all(m.scale == 1) and torch.all(m.scale_inv == 1)


@pytest.mark.parametrize("L,n,kind,fmt,margin", [
    (1, 1, 0, ops.FORMAT_HYBRID, 0),
    (16, 2, 0, ops.FORMAT_HYBRID, 0),
    (16, 1, 1, ops.FORMAT_HYBRID, 0),
    (16, 4, 0, ops.FORMAT_E4M3, 2),
    (1024, 4, 0, ops.FORMAT_E4M3, 0),
    (1024, 2, 1, ops.FORMAT_HYBRID, 1),
    (1024, 8, 1, ops.FORMAT_E5M2, 0),
    (37, 3, 1, ops.FORMAT_E4M3, 0),
])
def test_scaling_update_bit_exact(L, n, kind, fmt, margin):
    r = ops.Recipe(format=fmt, amax_history_len=L, margin=margin)
    m = ops.Meta(r, n, kind)
    om = oracle.Meta.fresh(L, [_fmt_of(r, kind)] * n)
    hist = inputs.random_history(L, n, inputs.seed_for("scaling", f"{L}/{n}/{kind}")).numpy()
    # adversarial entries: zero columns, inf, NaN, subnormal and huge amaxes
    if n > 1:
        hist[:, 0] = 0.0
    if L > 2:
        hist[1, n - 1] = np.inf if n > 2 else hist[1, n - 1]
        hist[L - 1, (n - 1) // 2] = np.nan
        hist[2 % L, min(1, n - 1)] = 1e-40
    m.history.copy_(torch.from_numpy(hist))
    om.history[:] = hist
    rng = np.random.default_rng(L * 31 + n)
    for step in range(6):
        ops.scaling_update(r, m)
        oracle.scaling_update(om, margin)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(m.history.cpu().numpy()), _bits(om.history))
        np.testing.assert_array_equal(_bits(m.scale.cpu().numpy()), _bits(om.scale))
        np.testing.assert_array_equal(_bits(m.scale_inv.cpu().numpy()), _bits(om.scale_inv))
        new = np.exp2(rng.uniform(-12, 12, size=n)).astype(np.float32)
        if step == 2:
            new[0] = np.float32(3e-39)      # scale overflows: kept
        m.history[0].copy_(torch.from_numpy(new))
        om.history[0] = new


@pytest.mark.parametrize("fmt,L,margin", [(ops.FORMAT_HYBRID, 1024, 0), (ops.FORMAT_E4M3, 16, 1)])
def test_scaling_update_batch_equals_one_by_one(fmt, L, margin):
    """70 state blocks of mixed kinds and slot counts (two launches of the batch)
    updated together and one at a time: identical histories, scales and scale_inv
    over four steps, with zero columns, inf, NaN and subnormal amaxes in them."""
    r = ops.Recipe(format=fmt, amax_history_len=L, margin=margin)
    shapes = [(1 + k % 4, k % 2) for k in range(70)]    # (slots, kind)
    one = [ops.Meta(r, n, kind) for n, kind in shapes]
    many = [ops.Meta(r, n, kind) for n, kind in shapes]
    rng = np.random.default_rng(L + margin)
    for k, ((n, _), a, b) in enumerate(zip(shapes, one, many)):
        hist = inputs.random_history(L, n, inputs.seed_for("batch", f"{k}")).numpy()
        if k % 5 == 0:
            hist[:, 0] = 0.0
        if k % 7 == 1:
            hist[L // 2, n - 1] = np.inf
        if k % 11 == 2:
            hist[L - 1, 0] = np.nan
        if k % 13 == 3:
            hist[0, n - 1] = 1e-40
        a.history.copy_(torch.from_numpy(hist))
        b.history.copy_(torch.from_numpy(hist))
    for step in range(4):
        for m in one:
            ops.scaling_update(r, m)
        ops.scaling_update_batch(r, many)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(one, many)):
            for x, y in ((a.history, b.history), (a.scale, b.scale), (a.scale_inv, b.scale_inv)):
                assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"step {step} block {k}"
        for (n, _), a, b in zip(shapes, one, many):
            new = torch.from_numpy(np.exp2(rng.uniform(-12, 12, size=n)).astype(np.float32))
            a.history[0].copy_(new)
            b.history[0].copy_(new)
