"""Quantization orders and the no-clip error bound.  TEST INFRASTRUCTURE ONLY.

Babai page, technical summary, 2.3 (error bound, the role of the order): without
clipping, the error of a row is bounded by a quarter of the scales weighted by the
diagonal D of the LDL factorisation of the reordered Hessian (Theorem 5); the bound
depends on the order, and a min-pivot order, choosing at every LDL step the smallest
remaining diagonal entry, makes the trace of D small; act order (descending Hessian
diagonal, quantized first) is the cheap approximation of it.

Reading (the page gives the rule, not its direction): the nearest-plane recursion
eliminates coordinates in the reverse of the quantization order (the column quantized
last is eliminated first, oracle.lattice.theorem5_bound), so
* the min-pivot elimination order picks, at each step, the remaining coordinate with
  the smallest Schur-complement diagonal, and GPTQ quantizes in the reverse of that
  order; among equal pivots the larger original index is eliminated first, so that in
  quantization order ties go to the smaller index, as in act order;
* with the raw diagonal in place of the Schur complements this is act order, which
  quantizes the largest diagonal first (ties to the smaller index).
Orders are returned as `perm`: perm[j] = the original column quantized j-th.
"""
from __future__ import annotations

import numpy as np


def act_order(H) -> np.ndarray:
    """Columns by descending H_jj, ties to the smaller index."""
    d = np.diag(np.asarray(H, np.float64))
    return np.lexsort((np.arange(d.shape[0]), -d)).astype(np.int64)


def min_pivot_order(H, hint=None, tol: float = 0.0):
    """Pivoted LDL by plain right-looking elimination in fp64, choosing the smallest
    current diagonal at each step.  Returns (perm, D, adopted): perm the quantization
    order (reverse of the elimination order), D[j] the LDL pivot of the column quantized
    j-th.  hint: another implementation's perm; at a step where the hinted column's
    current diagonal is within tol of the smallest, the hinted column is taken (a
    decision inside the rounding resolution), and such steps are counted."""
    A = np.array(H, np.float64)
    n = A.shape[0]
    remaining = list(range(n))
    elim, piv = [], []
    adopted = 0
    hint_elim = None if hint is None else np.asarray(hint)[::-1]
    for step in range(n):
        dvals = np.array([A[j, j] for j in remaining])
        m = dvals.min()
        k = remaining[int(np.flatnonzero(dvals == m)[-1])]  # ties: largest index first
        if hint_elim is not None:
            h = int(hint_elim[step])
            if h != k and h in remaining and A[h, h] <= m + tol:
                k = h
                adopted += 1
        p = A[k, k]
        elim.append(k)
        piv.append(p)
        remaining.remove(k)
        if remaining:
            r = np.array(remaining)
            col = A[r, k].copy()
            A[np.ix_(r, r)] -= np.outer(col, col) / p
    perm = np.array(elim[::-1], np.int64)
    D = np.array(piv[::-1])
    return perm, D, adopted


def schur_diagonal(H, eliminated, j) -> float:
    """H_jj - H_jP H_PP^{-1} H_Pj for the eliminated set P (linear solve, no elimination
    loop): the diagonal entry j after eliminating P."""
    H = np.asarray(H, np.float64)
    P = list(eliminated)
    if not P:
        return float(H[j, j])
    x = np.linalg.solve(H[np.ix_(P, P)], H[P, j])
    return float(H[j, j] - H[j, P] @ x)


def pivots_for_order(H, perm) -> np.ndarray:
    """LDL pivots of the column quantized j-th for a given quantization order: the
    diagonal of H reordered so the column quantized last is eliminated first."""
    from .lattice import ldl_diagonal
    elim = np.asarray(perm)[::-1]
    return ldl_diagonal(np.asarray(H, np.float64)[np.ix_(elim, elim)])[::-1]


def layer_bound(H, scale, group, perm) -> np.ndarray:
    """Per-row bound on f_r = 1/2 (w_r - q_r)^T H (w_r - q_r) without clipping in the
    given order: 1/8 sum_j D_j s_{r, g(perm_j)}^2 (Theorem 5 with f's factor 1/2)."""
    perm = np.asarray(perm)
    D = pivots_for_order(H, perm)
    s = np.asarray(scale, np.float64)[:, perm // group]     # [rows x d_i] in quantization order
    return 0.125 * (s * s) @ D
