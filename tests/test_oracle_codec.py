"""Pins for the oracle's bf16 / FP8 codec (CPU only).

The FP8 formats are named by the pages (HYBRID mixes E4M3 and E5M2) but defined
by the OCP 8-bit floating point specification; the closed forms below come
from the bit layouts (sign, exponent with bias, mantissa).  The encoder is
pinned against an independent brute-force nearest-value search.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import E4M3, E5M2


def brute_force_encode(values, fmt):
    """Nearest finite FP8 value by exhaustive search over the code table; an
    exact tie goes to the code whose last bit is 0.  NaN -> 0x7F, sign bit from
    the input's sign bit.  Nearest-finite search saturates by construction."""
    table = oracle.fp8_decode_table(fmt)
    codes = np.array([c for c in range(128) if np.isfinite(table[c])])
    vals = table[codes]
    v = np.asarray(values, dtype=np.float64).reshape(-1)
    out = np.empty(v.shape, dtype=np.uint8)
    for start in range(0, v.size, 4096):
        chunk = v[start:start + 4096]
        a = np.abs(np.where(np.isnan(chunk), 0.0, chunk))
        d = np.abs(a[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # Rounded distances can tie where the exact ones do not (huge |v|);
        # the exact nearest is always among the rounded-nearest, so those
        # rows are settled with exact rational arithmetic.
        # one nearest code: take it; several: resolve below
        pick = np.argmax(cand, axis=1)
        for i in np.nonzero((cand.sum(axis=1) > 1) | np.isinf(a))[0]:
            idx = np.nonzero(cand[i])[0]
            if np.isinf(a[i]):                 # every distance is infinite:
                idx = [len(codes) - 1]         # the largest finite value
            elif a[i] >= vals[idx].max():      # all candidates below |v|:
                idx = [idx.max()]              # the largest is the nearest
            else:
                ai = Fraction(float(a[i]))
                dist = [abs(ai - Fraction(float(vals[j]))) for j in idx]
                best = min(dist)
                idx = [j for j, dj in zip(idx, dist) if dj == best]
            even = [j for j in idx if codes[j] % 2 == 0]
            pick[i] = even[0] if even else idx[0]
        c = codes[pick].astype(np.uint8)
        c = c | np.where(np.signbit(chunk), 0x80, 0).astype(np.uint8)
        c = np.where(np.isnan(chunk), 0x7F, c)
        out[start:start + 4096] = c
    return out.reshape(np.shape(values))


# ---- closed forms from the OCP bit layouts ---------------------------------

def test_e4m3_closed_forms():
    t = oracle.fp8_decode_table(E4M3)
    assert t[0x7E] == (1 + 6 / 8) * 2.0 ** (15 - 7) == 448.0      # S.1111.110
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])                 # S.1111.111
    assert t[0x08] == 2.0 ** (1 - 7)                               # min normal 2^-6
    assert t[0x07] == (7 / 8) * 2.0 ** -6                          # max subnormal
    assert t[0x01] == 2.0 ** -9                                    # min subnormal
    assert t[0x38] == 1.0                                          # 0.0111.000
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0xFE] == -448.0
    assert not np.isinf(t).any()                                   # E4M3 has no inf


def test_e5m2_closed_forms():
    t = oracle.fp8_decode_table(E5M2)
    assert t[0x7B] == (1 + 3 / 4) * 2.0 ** (30 - 15) == 57344.0    # S.11110.11
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf                 # S.11111.00
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x04] == 2.0 ** -14                                   # min normal
    assert t[0x03] == (3 / 4) * 2.0 ** -14                         # max subnormal
    assert t[0x01] == 2.0 ** -16                                   # min subnormal
    assert t[0x3C] == 1.0                                          # 0.01111.00


@pytest.mark.parametrize("fmt,n_pos", [(E4M3, 127), (E5M2, 124)])
def test_decode_table_invariants(fmt, n_pos):
    t = oracle.fp8_decode_table(fmt)
    pos = oracle.fp8_positive_values(fmt)
    assert len(pos) == n_pos                       # finite non-negative values incl. 0
    assert np.all(np.diff(pos) > 0)                # strictly increasing with the code
    for c in range(128):                           # sign bit only flips the sign
        if np.isfinite(t[c]):
            assert t[c | 0x80] == -t[c]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_decode_roundtrip(fmt):
    t = oracle.fp8_decode_table(fmt)
    finite = [c for c in range(256) if np.isfinite(t[c])]
    codes = oracle.fp8_encode(t[finite], fmt)
    # -0 and +0 both round-trip to themselves
    assert list(codes) == finite


def test_encode_special_values_e4m3():
    enc = lambda v: int(oracle.fp8_encode(v, E4M3))
    assert enc(448.0) == 0x7E
    assert enc(-448.0) == 0xFE
    assert enc(464.0) == 0x7E          # midpoint to the (non-existent) 480: saturates
    assert enc(1e30) == 0x7E and enc(np.inf) == 0x7E and enc(-np.inf) == 0xFE
    assert enc(np.nan) == 0x7F and enc(-np.nan) == 0x7F
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00
    assert enc(2.0 ** -10) == 0x00     # half the min subnormal: tie -> even (0)
    assert enc(3 * 2.0 ** -10) == 0x02 # between 0x01 and 0x02: tie -> even
    assert enc(np.nextafter(2.0 ** -10, 1)) == 0x01
    assert enc(-1e-30) == 0x80         # tiny negatives keep the sign of zero
    assert enc(1.0625) == 0x38         # 1 + 1/16: tie between 1.0 and 1.125 -> even
    assert enc(1.1875) == 0x3A         # tie between 1.125 (0x39) and 1.25 (0x3A)


def test_encode_special_values_e5m2():
    enc = lambda v: int(oracle.fp8_encode(v, E5M2))
    assert enc(57344.0) == 0x7B
    assert enc(61440.0) == 0x7B        # midpoint to 65536 (inf code): saturates
    assert enc(np.inf) == 0x7B and enc(-np.inf) == 0xFB
    assert enc(np.nan) == 0x7F
    assert enc(2.0 ** -17) == 0x00     # tie -> even
    assert enc(3 * 2.0 ** -17) == 0x02
    assert enc(1.125) == 0x3C          # tie between 1.0 (0x3C) and 1.25 (0x3D) -> even


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encoder_matches_brute_force_on_all_bf16(fmt):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_to_f64(bits)
    np.testing.assert_array_equal(oracle.fp8_encode(v, fmt), brute_force_encode(v, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encoder_matches_brute_force_near_every_boundary(fmt):
    """Every float32 within 40 ulps of every rounding midpoint, of every
    representable value and of the saturation threshold, both signs."""
    pos = oracle.fp8_positive_values(fmt)
    anchors = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2, [pos[-1] * 1.5, 2 * pos[-1]]])
    anchors = anchors.astype(np.float32)
    ulps = np.arange(-40, 41, dtype=np.int64)
    bits = anchors.view(np.uint32).astype(np.int64)[:, None] + ulps[None, :]
    bits = bits[(bits >= 0) & (bits < 0x7F800000)].astype(np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    v = np.concatenate([v, -v])
    np.testing.assert_array_equal(oracle.fp8_encode(v, fmt), brute_force_encode(v, fmt))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encoder_matches_brute_force_on_random_float32(fmt):
    """Random sign and mantissa with the exponent field uniform below 2^30, plus
    a few fully random bit patterns (huge values, infinities, NaNs)."""
    rng = np.random.default_rng(7)
    n = 200_000
    sign = rng.integers(0, 2, size=n, dtype=np.uint64) << 31
    expo = rng.integers(0, 157, size=n, dtype=np.uint64) << 23
    mant = rng.integers(0, 1 << 23, size=n, dtype=np.uint64)
    bits = (sign | expo | mant).astype(np.uint32)
    wild = rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([bits, wild])
    with np.errstate(invalid="ignore"):
        v = bits.view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.fp8_encode(v, fmt), brute_force_encode(v, fmt))


def test_encoder_matches_brute_force_on_float64_between_float32():
    """The oracle encodes float64 products; check values that are not float32."""
    rng = np.random.default_rng(11)
    v = rng.normal(size=100_000) * np.exp2(rng.uniform(-20, 18, size=100_000))
    for fmt in (E4M3, E5M2):
        np.testing.assert_array_equal(oracle.fp8_encode(v, fmt), brute_force_encode(v, fmt))


# ---- bf16 ----------------------------------------------------------------

def test_bf16_decode_is_exact_top_half_of_float32():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    np.testing.assert_array_equal(np.isnan(v), torch.isnan(ref).numpy())
    ok = ~np.isnan(v)
    np.testing.assert_array_equal(v[ok], ref.numpy()[ok])


def test_bf16_rounding_matches_torch_on_float32_inputs():
    """For float32 inputs torch's float -> bf16 conversion is one RNE rounding."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=300_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    ours = oracle.f64_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_ties_and_specials():
    b = lambda v: int(oracle.f64_to_bf16_bits(v))
    assert b(1.0) == 0x3F80
    assert b(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even
    assert b(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert b(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81   # just above the tie (float64 only)
    assert b(-0.0) == 0x8000
    assert b(np.inf) == 0x7F80 and b(-np.inf) == 0xFF80
    assert b(np.nan) == 0x7FC0
    assert b(3.5e38) == 0x7F80                     # past the largest finite bf16
