"""Pins for the oracle's delayed-scaling bookkeeping (CPU only).

The pages fix a per-tensor scale, a 2-D amax history with the newest amaxes in
row 0, history lengths 16 and 1024 and the "max" reduction (tutorial setup and
benchmark listings; "Turbo-charging ...", "Playing with lower-precision
formats").  The scale formula fp8_max / max(history) / 2^margin is this
path's reading; the checks below pin the oracle to it with exact rational
arithmetic and to the history's window semantics with a brute-force FIFO.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import E4M3, E5M2, Meta


def nearest_f32(x: Fraction) -> np.float32:
    """Correctly rounded binary32 value of a positive rational (ties to even),
    found by bracketing with float64 and checking the neighbours exactly."""
    guess = np.float32(float(x))
    cands = {guess, np.nextafter(guess, np.float32(0)), np.nextafter(guess, np.float32(np.inf))}
    cands = sorted(c for c in cands if np.isfinite(c))
    best = min(abs(Fraction(float(c)) - x) for c in cands)
    tied = [c for c in cands if abs(Fraction(float(c)) - x) == best]
    if len(tied) > 1:
        tied = [c for c in tied if (int(np.array(c).view(np.uint32)) & 1) == 0]
    return np.float32(tied[0])


def fresh(L, fmts):
    return Meta.fresh(L, fmts)


@pytest.mark.parametrize("fmt,amax,margin,expected", [
    (E4M3, 448.0, 0, 1.0),
    (E4M3, 1.0, 0, 448.0),
    (E4M3, 1.0, 1, 224.0),
    (E4M3, 2.0, 3, 28.0),
    (E4M3, 0.5, 0, 896.0),
    (E5M2, 57344.0, 0, 1.0),
    (E5M2, 1.0, 0, 57344.0),
    (E5M2, 7.0, 0, 8192.0),
])
def test_scale_closed_forms(fmt, amax, margin, expected):
    m = fresh(4, [fmt])
    m.history[0, 0] = amax
    oracle.scaling_update(m, margin)
    assert m.scale[0] == np.float32(expected)
    assert m.scale_inv[0] == np.float32(1.0 / expected)


@pytest.mark.parametrize("bad", [0.0, np.inf, np.nan, 1e-40])
def test_scale_kept_when_amax_unusable(bad):
    """amax 0, inf or NaN, or a subnormal amax whose scale overflows: keep the
    previous scale (the initial one is 1)."""
    m = fresh(2, [E4M3])
    m.history[0, 0] = bad
    oracle.scaling_update(m)
    assert m.scale[0] == 1.0 and m.scale_inv[0] == 1.0
    # a usable amax later in the window updates it; the unusable one must leave first
    m.history[0, 0] = 2.0
    oracle.scaling_update(m)
    if np.isnan(bad) or np.isinf(bad):
        assert m.scale[0] == 1.0                  # bad value still in the window
        oracle.scaling_update(m)                  # it has now rolled out
    assert m.scale[0] == np.float32(224.0)


def test_scale_is_correctly_rounded_binary32_division():
    rng = np.random.default_rng(5)
    amaxes = np.exp2(rng.uniform(-30, 30, size=2000)).astype(np.float32)
    for fmt in (E4M3, E5M2):
        for margin in (0, 2):
            for a in amaxes:
                m = fresh(1, [fmt])
                m.history[0, 0] = a
                oracle.scaling_update(m, margin)
                exact = Fraction(int(oracle.FP8_MAX[fmt])) / Fraction(float(a))
                want = nearest_f32(exact)
                if not np.isfinite(want):
                    assert m.scale[0] == 1.0
                    continue
                want = np.float32(np.ldexp(want, -margin))
                assert m.scale[0] == want, (fmt, margin, a)
                assert m.scale_inv[0] == nearest_f32(1 / Fraction(float(m.scale[0])))


@pytest.mark.parametrize("L", [1, 2, 16, 1024])
def test_history_is_a_window_of_the_last_L_amaxes(L):
    """Brute-force FIFO: after step t's update, the scale comes from the
    largest of the amaxes of steps t-L .. t-1 and row i holds step t-1-i's
    amax (row 0 is then cleared for step t)."""
    rng = np.random.default_rng(L)
    m = fresh(L, [E4M3, E5M2])
    seen = []                         # amaxes recorded so far, oldest first
    for step in range(2 * L + 3 if L < 1024 else L + 3):
        oracle.scaling_update(m)
        window = seen[-L:]
        for s, fmt in enumerate((E4M3, E5M2)):
            if window:
                a = max(w[s] for w in window)
                want = nearest_f32(Fraction(int(oracle.FP8_MAX[fmt])) / Fraction(float(a)))
                assert m.scale[s] == want
            else:
                assert m.scale[s] == 1.0
        # after the roll: row 0 is zero, row i (i >= 1) is step-i's amax
        expect = np.zeros((L, 2), dtype=np.float32)
        for i in range(1, min(L, step + 1)):
            expect[i] = seen[step - i]
        assert np.array_equal(m.history, expect)
        amax = rng.uniform(0.5, 100.0, size=2).astype(np.float32)
        m.history[0] = amax
        seen.append(amax)


def test_history_len_1_is_previous_step_amax():
    m = fresh(1, [E4M3])
    for a in (3.0, 7.0, 0.25):
        m.history[0, 0] = a
        oracle.scaling_update(m)
        assert m.scale[0] == np.float32(448.0 / a)


def test_scale_inv_times_scale_is_one_within_an_ulp():
    rng = np.random.default_rng(9)
    for a in np.exp2(rng.uniform(-20, 20, size=500)).astype(np.float32):
        m = fresh(1, [E4M3])
        m.history[0, 0] = a
        oracle.scaling_update(m)
        prod = Fraction(float(m.scale[0])) * Fraction(float(m.scale_inv[0]))
        assert abs(prod - 1) <= Fraction(1, 2 ** 23)


def test_record_amax_keeps_max_and_nan():
    m = fresh(4, [E4M3])
    m.record_amax(0, np.float32(2.0))
    m.record_amax(0, np.float32(1.0))
    assert m.history[0, 0] == 2.0
    m.record_amax(0, np.float32(np.nan))
    m.record_amax(0, np.float32(5.0))
    assert np.isnan(m.history[0, 0])


def test_recipe_fixture_matches_oracle_defaults():
    """tests/golden/recipe.txt: the recipe values the pages print."""
    import os
    rows = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "recipe.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            rows.setdefault(k, []).append(v)
    r = oracle.Recipe()
    assert rows["format"] == ["HYBRID"] and r.format == oracle.FORMAT_HYBRID
    assert int(rows["amax_history_len"][0]) == r.amax_history_len == 16
    assert int(rows["amax_history_len_alt"][0]) == 1024
    assert rows["amax_compute_algo"] == ["max"]
    assert set(rows["format_variant"]) == {"E4M3", "E5M2"}
    # HYBRID: E4M3 forward, E5M2 backward; E4M3 recipe: E4M3 both ways
    assert oracle.fwd_format(r) == E4M3 and oracle.bwd_format(r) == E5M2
    r4 = oracle.Recipe(format=oracle.FORMAT_E4M3)
    assert oracle.fwd_format(r4) == E4M3 and oracle.bwd_format(r4) == E4M3
