"""Quantization grid and round-to-nearest (RTN).  TEST INFRASTRUCTURE ONLY.

The set Q of the ADMM-Q page (technical summary, 1. problem formulation) is a
b-bit asymmetric grid per (output row, group of g consecutive input columns):
value(c) = s (c - z), c in {0, ..., 2^b - 1}.  The pages fix neither the fit
rule nor the rounding; the readings used here are

* range: lo = min(min v, 0), hi = max(max v, 0) over the group (the range is forced
  to hold 0 so that the integer zero point fits in b bits, as the GPTQ storage
  format that ADMM-Q keeps needs -- ADMM-Q page, experiments, 3. inference);
  an all-zero group uses [-1, 1];
* s = (hi - lo) / (2^b - 1),  z = clamp(rint(-lo / s), 0, 2^b - 1);
* code(x) = clamp(rint(x / s) + z, 0, 2^b - 1), rint = round half to even
  (RTN: every weight rounded to the nearest grid point on its own -- ADMM-Q page,
  problem statement; the clamp is the "clipping" of the Babai page, section 3).

The fit and the RTN used for the static grid run in IEEE fp32 (numpy float32 is
correctly rounded), so the GPU library must match them bit for bit.  Inside the
fp64 solvers the same rounding runs on fp64 pre-round values, with an optional
boundary rule: where the pre-round value x/s lies within `tol` of a half-integer,
both neighbouring codes are acceptable and a supplied hint picks one.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def maxq(bits: int) -> int:
    return (1 << bits) - 1


def fit_range_f32(v: np.ndarray, group: int):
    """Per-(row, group) range [lo, hi] of fp32 values v [rows x cols], forced to
    contain 0; an all-zero group becomes [-1, 1].  Returns fp32 arrays [rows x G]."""
    v = np.asarray(v, dtype=F32)
    rows, cols = v.shape
    assert cols % group == 0
    vg = v.reshape(rows, cols // group, group)
    lo = np.minimum(vg.min(axis=2), F32(0))
    hi = np.maximum(vg.max(axis=2), F32(0))
    deg = hi == lo
    lo = np.where(deg, F32(-1), lo).astype(F32)
    hi = np.where(deg, F32(1), hi).astype(F32)
    return lo, hi


def grid_from_range_f32(lo: np.ndarray, hi: np.ndarray, bits: int):
    """s = fl32(fl32(hi - lo) / (2^b - 1)), z = clamp(rint(fl32(-lo / s)), 0, 2^b-1)."""
    lo = np.asarray(lo, dtype=F32)
    hi = np.asarray(hi, dtype=F32)
    q = F32(maxq(bits))
    s = ((hi - lo) / q).astype(F32)
    z = np.clip(np.rint((-lo / s).astype(F32)), F32(0), q).astype(np.uint8)
    return s, z


def fit_grid_f32(v: np.ndarray, bits: int, group: int):
    """Static grid of the weights v (fp32 [rows x cols]): (scale f32, zero u8), [rows x G]."""
    lo, hi = fit_range_f32(v, group)
    return grid_from_range_f32(lo, hi, bits)


def rtn_f32(v: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int, group: int):
    """Round-to-nearest codes in IEEE fp32: clamp(rint(fl32(x / s)) + z, 0, 2^b - 1)."""
    v = np.asarray(v, dtype=F32)
    rows, cols = v.shape
    s = np.repeat(np.asarray(scale, F32), group, axis=1)
    z = np.repeat(np.asarray(zero).astype(F32), group, axis=1)
    u = np.rint((v / s).astype(F32)) + z
    return np.clip(u, F32(0), F32(maxq(bits))).astype(np.uint8)


def dequant(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """fp64 grid values s (c - z) for codes [rows x cols] on a per-group grid."""
    s = np.repeat(np.asarray(scale, np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, np.float64), group, axis=1)
    return s * (np.asarray(codes, np.float64) - z)


def round_codes(u: np.ndarray, z, bits: int, clip: bool = True, hint=None, tol: float = 1e-4):
    """Codes from fp64 pre-round values u = x / s (code units, zero point not yet
    added): c = rint(u) + z, clamped to [0, 2^b - 1] when `clip`.

    Boundary rule: where u lies within `tol` of a half-integer, the two codes on
    either side are both acceptable; if `hint` (same shape) holds one of them, it is
    taken.  Returns (codes int64, number of hint adoptions, mask of near-boundary
    elements)."""
    u = np.asarray(u, np.float64)
    z = np.asarray(z, np.float64)
    c = np.rint(u) + z
    if clip:
        c = np.clip(c, 0, maxq(bits))
    near = np.abs(u - np.floor(u) - 0.5) <= tol
    adopted = 0
    if hint is not None and near.any():
        h = np.asarray(hint, np.float64)
        lo_c = np.floor(u) + z
        hi_c = lo_c + 1
        if clip:
            lo_c = np.clip(lo_c, 0, maxq(bits))
            hi_c = np.clip(hi_c, 0, maxq(bits))
        ok = near & ((h == lo_c) | (h == hi_c)) & (h != c)
        adopted = int(ok.sum())
        c = np.where(ok, h, c)
    return c.astype(np.int64), adopted, near


def fit_range_f64(v: np.ndarray, group: int):
    """fp64 version of fit_range_f32 (used by the ADMM grid refresh)."""
    v = np.asarray(v, dtype=np.float64)
    rows, cols = v.shape
    vg = v.reshape(rows, cols // group, group)
    lo = np.minimum(vg.min(axis=2), 0.0)
    hi = np.maximum(vg.max(axis=2), 0.0)
    deg = hi == lo
    return np.where(deg, -1.0, lo), np.where(deg, 1.0, hi)


def grid_from_range_f64(lo, hi, bits: int, zero_hint=None, tol: float = 1e-4):
    """Grid from an fp64 range: s is stored in fp32 (the storage format keeps fp32
    scales), rounded from the fp64 quotient; z = clamp(rint(-lo / s)) with the same
    boundary rule as round_codes.  Returns (s f32, z int64, adoptions)."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    s = ((hi - lo) / maxq(bits)).astype(F32)
    u = -lo / s.astype(np.float64)
    z, n, _ = round_codes(u, 0.0, bits, True, zero_hint, tol)
    return s, z, n
