"""Comparison rules between the HIP path and the oracle (test helpers).

* FP8 codes: the GPU code must encode a value within a window of the oracle's
  exact value v.  For a LayerNorm output the window is
  1e-6 * max(|v|, scale * (|gamma * xhat| + |beta|)) (the second term covers the
  cancellation between gamma * xhat and beta), which allows a one-step difference
  only next to a rounding midpoint; casts of bf16/fp32 tensors are exact (window
  0); a GEMM-fed cast (GELU of fc1) gets the GEMM's own error bound.
* GEMM-shaped outputs: max_ij |gpu - oracle| / ||oracle row i||_2 <= 2e-2, and an
  alarm on the per-row relative L2 error (catches a dropped K tile or a wrong
  epilogue term, which move rows by O(1)).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def to_np_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns (on the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(to_np_bits(t))
    return t.detach().cpu().numpy()


def signed_index(codes: np.ndarray) -> np.ndarray:
    """Position of each code in value order; +0 and -0 both map to 0."""
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def midpoint_distance(v: np.ndarray, fmt: str):
    """(distance from |v| to the nearest rounding midpoint, that midpoint)."""
    pos = oracle.fp8_positive_values(fmt)
    mids = (pos[:-1] + pos[1:]) / 2
    a = np.abs(v)
    i = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    d_lo = np.abs(a - mids[i - 1])
    d_hi = np.abs(mids[i] - a)
    near = np.where(d_lo < d_hi, mids[i - 1], mids[i])
    return np.minimum(d_lo, d_hi), near


def compare_codes(gpu_codes: np.ndarray, exact: np.ndarray, fmt: str, window):
    """Check FP8 codes against the oracle.

    exact: the oracle's value before encoding (float64); window: the absolute
    error bound of the HIP path's value.  The GPU code must be the encoding of
    some value within [exact - window, exact + window]: with a window far below
    the code spacing this is "equal, or one step off where the exact value lies
    within the window of a rounding midpoint"; window 0 demands equality.  +0 and
    -0 count as the same value; NaN must give 0x7F.  Returns counts; raises
    AssertionError on a violation."""
    gpu_codes = np.asarray(gpu_codes, dtype=np.uint8).reshape(-1)
    exact = np.asarray(exact, dtype=np.float64).reshape(-1)
    window = np.asarray(window, dtype=np.float64)
    window = window.reshape(-1) if window.size == exact.size else \
        np.broadcast_to(window, exact.shape).reshape(-1)
    ref = oracle.fp8_encode(exact, fmt)
    nan = np.isnan(exact)
    assert np.all(gpu_codes[nan] == 0x7F), "NaN inputs must encode to 0x7F"
    gi, ri = signed_index(gpu_codes), signed_index(ref)
    lo = signed_index(oracle.fp8_encode(exact - window, fmt))
    hi = signed_index(oracle.fp8_encode(exact + window, fmt))
    bad = ((gi < lo) | (gi > hi)) & ~nan
    diff = (gi != ri) & ~nan
    if bad.any():
        idx = np.nonzero(bad)[0][:8]
        dist, _ = midpoint_distance(exact[idx], fmt)
        raise AssertionError(
            f"{int(bad.sum())} FP8 codes outside the rule; first at {idx.tolist()}: "
            f"gpu={gpu_codes[idx].tolist()} oracle={ref[idx].tolist()} "
            f"exact={exact[idx].tolist()} midpoint distance={dist.tolist()} "
            f"window={window[idx].tolist()}")
    return dict(n=int(exact.size), mismatched=int(diff.sum()),
                near_boundary=int(((lo != ri) | (hi != ri)).sum()))


def ln_window(gamma_xhat: np.ndarray, beta: np.ndarray, scale: float, exact: np.ndarray):
    """The LayerNorm-output window: 1e-6 * max(|v|, s (|gamma xhat| + |beta|)),
    with |v| standing in for the midpoint it is being compared with."""
    mag = float(scale) * (np.abs(gamma_xhat) + np.abs(beta))
    return 1e-6 * np.maximum(np.abs(exact), mag)


def gemm_rel_error(gpu: np.ndarray, ref: np.ndarray):
    """(max_ij |d_ij| / ||ref_i||, max_i ||d_i|| / ||ref_i||) over rows with a
    non-zero reference."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    norms = np.linalg.norm(ref, axis=1)
    ok = norms > 0
    d = np.abs(gpu - ref)
    if not ok.any():
        return float(d.max(initial=0.0)), float(d.max(initial=0.0))
    a = (d[ok].max(axis=1) / norms[ok]).max()
    b = (np.linalg.norm(d[ok], axis=1) / norms[ok]).max()
    zero_rows = ~ok
    if zero_rows.any():
        a = max(a, d[zero_rows].max())
        b = max(b, d[zero_rows].max())
    return float(a), float(b)


def assert_gemm_close(gpu, ref, tol=2e-2, alarm=2e-2, what="output"):
    """The GEMM rule plus an alarm on each row's relative L2 error.  A one-step
    FP8 code difference that the code rule allows moves a whole output row by up
    to ~1e-2 in relative L2, so the alarm is only tightened where no code can
    differ (operands given as codes)."""
    a, b = gemm_rel_error(gpu, ref)
    assert a <= tol, f"{what}: max |d| / row norm = {a:.3e} > {tol}"
    assert b <= alarm, f"{what}: row relative L2 error = {b:.3e} > {alarm}"
    return a, b


def assert_vector_close(gpu, ref, tol, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e = np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)
    assert e <= tol, f"{what}: relative L2 error {e:.3e} > {tol}"
    return e


def compare_bf16(gpu_bits, exact, window):
    """bf16 outputs of an fp32 computation against the float64 result: each GPU
    value must lie between the roundings of exact - window and exact + window
    (rounding is monotone), so it equals the rounding of exact except next to a
    rounding midpoint, where the neighbour is allowed.  Returns counts."""
    g = oracle.bf16_to_f64(np.asarray(gpu_bits, dtype=np.uint16).reshape(-1))
    exact = np.asarray(exact, dtype=np.float64).reshape(-1)
    window = np.broadcast_to(np.asarray(window, dtype=np.float64).reshape(-1)
                             if np.size(window) == exact.size else window, exact.shape)
    lo = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(exact - window))
    hi = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(exact + window))
    ref = oracle.bf16_to_f64(oracle.f64_to_bf16_bits(exact))
    bad = (g < lo) | (g > hi)
    if bad.any():
        idx = np.nonzero(bad)[0][:8]
        raise AssertionError(f"{int(bad.sum())} bf16 values outside the rule; first at "
                             f"{idx.tolist()}: gpu={g[idx].tolist()} exact={exact[idx].tolist()}")
    return dict(n=int(exact.size), mismatched=int((g != ref).sum()),
                near_boundary=int(((lo != ref) | (hi != ref)).sum()))
