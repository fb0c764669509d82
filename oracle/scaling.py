"""Delayed-scaling bookkeeping (oracle, test infrastructure only).

What the pages fix: the recipe keeps, per module, a per-tensor scale vector and
a 2-D amax history whose row 0 holds the most recent amaxes (tutorial,
benchmark listing: fp8_meta["scaling_fwd"].scale and .amax_history[0, :4]);
the history length is 16 or 1024 and the history is reduced with "max"
(tutorial setup listing and "things to try"); the scale tracks the amax of
each tensor "on the fly" so the FP8 values do not overflow ("Turbo-charging
...", "Playing with lower-precision formats: BF16 vs FP8").

Readings taken where the pages are silent:

* scale = fp8_max / max(history) / 2^margin, computed as one IEEE binary32
  division followed by an exact power-of-two scaling; fp8_max is 448 for an
  E4M3 tensor and 57344 for an E5M2 tensor; margin is an integer >= 0.
* If max(history) is zero, not finite (inf or NaN anywhere in the window) or
  the new scale is not a positive finite number, the previous scale is kept.
  A fresh module starts with an all-zero history and scale = scale_inv = 1.
* scale_inv = 1 / scale as one binary32 division.
* The update runs at the start of a step: reduce all rows, then shift every
  row down by one (the oldest row falls off), then zero row 0.  The step's
  kernels then record their amaxes into row 0.  So step t is scaled from the
  amaxes of steps t-L .. t-1, never from its own (delayed scaling).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .codec import E4M3, E5M2, FP8_MAX


def fp8_max_for(fmt: str) -> np.float32:
    return np.float32(FP8_MAX[fmt])


@dataclass
class Meta:
    """One module's FP8 state for one direction (forward or backward).

    history: float32 [L][n_slots], row 0 newest; scale, scale_inv: float32
    [n_slots]; formats: the FP8 format of each slot's tensor."""
    history: np.ndarray
    scale: np.ndarray
    scale_inv: np.ndarray
    formats: list = field(default_factory=list)

    @classmethod
    def fresh(cls, history_len: int, formats) -> "Meta":
        n = len(formats)
        return cls(history=np.zeros((history_len, n), dtype=np.float32),
                   scale=np.ones(n, dtype=np.float32),
                   scale_inv=np.ones(n, dtype=np.float32),
                   formats=list(formats))

    def copy(self) -> "Meta":
        return Meta(self.history.copy(), self.scale.copy(), self.scale_inv.copy(),
                    list(self.formats))

    def record_amax(self, slot: int, amax: np.float32) -> None:
        """Row 0 keeps the largest amax recorded this step (NaN wins)."""
        cur = self.history[0, slot]
        a = np.float32(amax)
        if np.isnan(a) or np.isnan(cur):
            self.history[0, slot] = np.float32(np.nan)
        else:
            self.history[0, slot] = max(cur, a)


def scaling_update(meta: Meta, margin: int = 0) -> None:
    """Update scale and scale_inv from the history, then roll it (in place)."""
    hist = meta.history
    L, n = hist.shape
    for s in range(n):
        col = hist[:, s]
        a = np.float32(np.nan) if np.isnan(col).any() else np.float32(col.max())
        if np.isfinite(a) and a > 0:
            with np.errstate(over="ignore", divide="ignore"):
                new = fp8_max_for(meta.formats[s]) / a                   # binary32 division
                new = np.float32(np.ldexp(new, -int(margin)))            # exact 2^-margin
            if np.isfinite(new) and new > 0:
                meta.scale[s] = new
        with np.errstate(over="ignore", divide="ignore"):
            meta.scale_inv[s] = np.float32(1.0) / meta.scale[s]
    # roll: row i <- row i-1, row 0 <- 0
    if L > 1:
        hist[1:, :] = hist[:-1, :].copy()
    hist[0, :] = 0.0
