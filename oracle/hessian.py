"""Calibration Hessian.  TEST INFRASTRUCTURE ONLY.

ADMM-Q page, technical summary 1. problem formulation: H = X^T X + lambda I with X the
calibration activations [tokens x d_i].  The GPTQ tutorial page (section 2) writes
the per-row curvature as 2 X X^T with X stored [d_i x tokens]; the factor 2 is dropped
here (it changes neither the minimiser nor the damping relative to the diagonal).

Readings: lambda = damp * mean(diag(X^T X)), taken on the undamped diagonal and added
once (the GPTQ tutorial's damping section asks only for a positive diagonal shift that
keeps small eigenvalues away from zero); Sigma = Diag(H)^(-1/2) and the scaled
H~ = Sigma H Sigma (ADMM-Q page, key components, "diagonal scaling").

All sums run in fp64 on the exact values of the bf16 (or fp32) inputs.
"""
from __future__ import annotations

import numpy as np

from .grid import F32


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(F32).astype(np.float64)


def gram(X, chunk: int = 8192) -> np.ndarray:
    """X^T X = sum over tokens t of x_t x_t^T, evaluated in fp64 over token slices
    (slicing only bounds memory; the sum is the definition).  X: fp32/fp64 array,
    or uint16 bf16 bit patterns."""
    n, d = X.shape
    G = np.zeros((d, d))
    for a in range(0, n, chunk):
        xs = X[a:a + chunk]
        xs = bf16_to_f64(xs) if xs.dtype == np.uint16 else np.asarray(xs, np.float64)
        G += xs.T @ xs
    return G


def damping(G: np.ndarray, damp: float) -> float:
    """lambda = damp * mean(diag(X^T X))."""
    return float(damp * np.mean(np.diag(G)))


def hessian(X, damp: float):
    """H = X^T X + lambda I; returns (H, lambda)."""
    G = gram(X)
    lam = damping(G, damp)
    return G + lam * np.eye(G.shape[0]), lam


def scaling(H: np.ndarray):
    """Sigma = Diag(H)^(-1/2) as a vector, and H~ = Sigma H Sigma (unit diagonal)."""
    d = np.diag(H).astype(np.float64)
    sig = 1.0 / np.sqrt(d)
    return sig, H * sig[:, None] * sig[None, :]


def gram_entries(X, ii: np.ndarray, jj: np.ndarray) -> np.ndarray:
    """Selected entries (X^T X)[ii, jj] as fp64 dot products over all tokens."""
    xi = X[:, ii]
    xj = X[:, jj]
    if X.dtype == np.uint16:
        xi, xj = bf16_to_f64(xi), bf16_to_f64(xj)
    else:
        xi, xj = np.asarray(xi, np.float64), np.asarray(xj, np.float64)
    return np.einsum("ti,ti->i", xi, xj)
