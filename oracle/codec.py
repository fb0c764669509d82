"""bf16 and FP8 number formats (oracle, test infrastructure only).

The tutorial's recipe uses HYBRID ("mixes E4M3 and E5M2") and names Format.E4M3
("Turbo-charging ...", "Playing with lower-precision formats: BF16 vs FP8";
tutorial setup listing).  Neither page gives the bit layouts, so this file
takes them from the OCP 8-bit floating point specification (OFP8):

* E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.  No infinities;
  S.1111.111 is NaN, so the largest finite value is S.1111.110 = 1.75 * 2^8
  = 448.  Subnormals are m * 2^-9.
* E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like:
  S.11111.00 is infinity, S.11111.{01,10,11} are NaN, the largest finite value
  is S.11110.11 = 1.75 * 2^15 = 57344.  Subnormals are m * 2^-16.

The encoder rounds to nearest with ties to the even code (mantissa LSB 0),
saturates anything beyond the largest finite value (infinities included) to
it, keeps the sign of zero and maps every NaN to 0x7F.  Saturation is the
reading that keeps an overflowing scaled value finite; the pages only say
that delayed scaling exists to prevent overflow.

bf16 values are the top 16 bits of an IEEE binary32 value.
"""
from __future__ import annotations

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"

FP8_MAX = {E4M3: 448.0, E5M2: 57344.0}

# largest finite bf16 value: (2 - 2^-7) * 2^127
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127

_LAYOUT = {
    # format: (exponent bits, mantissa bits, bias)
    E4M3: (4, 3, 7),
    E5M2: (5, 2, 15),
}


def _decode_one(code: int, fmt: str) -> float:
    ebits, mbits, bias = _LAYOUT[fmt]
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    emax_field = (1 << ebits) - 1
    if fmt == E4M3 and e == emax_field and m == (1 << mbits) - 1:
        return float("nan")
    if fmt == E5M2 and e == emax_field:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        # subnormal: 0.m * 2^(1 - bias)
        return sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


_TABLES = {fmt: np.array([_decode_one(c, fmt) for c in range(256)], dtype=np.float64)
           for fmt in (E4M3, E5M2)}


def fp8_decode_table(fmt: str) -> np.ndarray:
    """float64 value of each of the 256 codes (a copy)."""
    return _TABLES[fmt].copy()


def fp8_decode(codes, fmt: str) -> np.ndarray:
    """Decode uint8 codes to float64 (exact)."""
    return _TABLES[fmt][np.asarray(codes, dtype=np.uint8)]


def fp8_positive_values(fmt: str) -> np.ndarray:
    """The finite non-negative values, indexed by code 0x00 .. largest finite code."""
    t = _TABLES[fmt]
    max_code = int(np.nonzero(t[:128] == FP8_MAX[fmt])[0][0])
    return t[:max_code + 1].copy()


def fp8_encode(values, fmt: str) -> np.ndarray:
    """Round float64 values to FP8 codes: nearest, ties to even, saturating,
    signed zero kept, NaN -> 0x7F."""
    v = np.asarray(values, dtype=np.float64)
    pos = fp8_positive_values(fmt)
    max_code = len(pos) - 1
    a = np.abs(v)
    nan = np.isnan(v)
    a_safe = np.where(nan, 0.0, a)
    # lo: largest code whose value is <= |v|
    lo = np.searchsorted(pos, a_safe, side="right") - 1
    lo = np.clip(lo, 0, max_code)
    hi = np.minimum(lo + 1, max_code)
    mid = (pos[lo] + pos[hi]) * 0.5          # exact: both are short binary fractions
    pick_hi = a_safe > mid
    tie = a_safe == mid
    pick_hi = np.where(tie & (lo != hi), (lo & 1) == 1, pick_hi)  # tie -> even code
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a_safe >= FP8_MAX[fmt], max_code, mag)     # saturate (incl. inf)
    code = mag.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    code = np.where(nan, 0x7F, code).astype(np.uint8)
    return code


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(values) -> np.ndarray:
    """float64 -> bf16 bit patterns with one rounding to nearest, ties to even.

    bf16 keeps 8 significant bits, so for v = m * 2^e (0.5 <= |m| < 1) the
    spacing is 2^(e-8), floored at the subnormal spacing 2^-133.  Results past
    the largest finite bf16 value become infinities; NaN becomes 0x7FC0."""
    v = np.asarray(values, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(v)
        q = np.maximum(e - 8, -133)
        r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)
        bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)
