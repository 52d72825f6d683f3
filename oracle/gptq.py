"""GPTQ, two independent routes.  TEST INFRASTRUCTURE ONLY.

Both routes quantize the columns of W [d_o x d_i] one at a time in a common order
shared by every row, each row against its own static grid (the grid is an input of
the algorithm: GPTQ tutorial page, section 3, Algorithm 1 inputs; the ADMM-Q page's
grid-refresh item notes that GPTQ keeps the grid fixed).

* gptq_plain -- the definition.  GPTQ tutorial page, section 2, "a Lagrange multiplier
  gives the compensation direction": fixing coordinate q to its grid value changes it
  by d; the free coordinates move by -d H_F^{-1} e_q / (H_F^{-1})_qq, where H_F^{-1} is
  the inverse curvature of the still-free coordinates, after which q leaves the free
  set (the rank-one downdate of the inverse).
* gptq -- the same compensation written with the factor of section 3: R upper with
  R^T R = H^{-1}.  Row j of R, divided by R_jj, is the compensation direction of
  section 2 once the columns before j have left the free set (the successive
  downdates of the inverse are what the Cholesky factorisation of H^{-1} computes,
  one row at a time), so column k, when its turn comes, holds its original value
  minus everything the earlier columns sent it:
      w_k = w_hat_k - sum_{j<k} E_j R_jk,   E_j = (w_j - q_j) / R_jj.
  This route forms that sum directly for each column (left-looking).  The tutorial's
  blocks of B columns with one matrix-product update of the later columns per block
  (section 3) regroup the same terms, so the block size does not enter here; tests
  check a blocked evaluation against this one.

H passed here already holds the damping (the Hessian builder adds lambda I once).
"""
from __future__ import annotations

import numpy as np

from .grid import round_codes


def inverse_factor(H: np.ndarray) -> np.ndarray:
    """Upper-triangular R with R^T R = H^{-1}: invert, then take the Cholesky factor
    (GPTQ tutorial page, section 3: R = upper Cholesky((H + lambda I)^{-1}))."""
    Hinv = np.linalg.inv(np.asarray(H, np.float64))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def inverse_factor_lapack(H: np.ndarray) -> np.ndarray:
    """The same R as inverse_factor (invert, then the upper Cholesky factor of the
    inverse), through LAPACK's symmetric positive-definite drivers: H = U^T U (potrf),
    H^{-1} from U (potri), then R^T R = H^{-1} (potrf).  About a third of the general
    inverse's work, for layers with tens of thousands of input channels."""
    from scipy.linalg import lapack
    A = np.array(H, np.float64, order="F")
    U, info = lapack.dpotrf(A, lower=0, clean=1, overwrite_a=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"H is not positive definite (potrf info {info})")
    Hinv, info = lapack.dpotri(U, lower=0, overwrite_c=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"potri info {info}")
    iu = np.triu_indices_from(Hinv, 1)
    Hinv[(iu[1], iu[0])] = Hinv[iu]
    R, info = lapack.dpotrf(Hinv, lower=0, clean=1, overwrite_a=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"H^-1 is not positive definite (potrf info {info})")
    return np.ascontiguousarray(R)


def _column_grid(scale, zero, group, col):
    g = col // group
    return np.asarray(scale[:, g], np.float64), np.asarray(zero[:, g], np.float64)


def gptq_plain(H, W_hat, scale, zero, bits, group, order=None, clip=True):
    """Lagrange / rank-one-downdate route.  Returns integer codes [d_o x d_i] in the
    original column positions."""
    W = np.array(W_hat, np.float64)
    d_o, d_i = W.shape
    order = np.arange(d_i) if order is None else np.asarray(order)
    Hinv = np.linalg.inv(np.asarray(H, np.float64))
    free = list(order)
    codes = np.zeros((d_o, d_i), np.int64)
    for col in order:
        s, z = _column_grid(scale, zero, group, col)
        c, _, _ = round_codes(W[:, col] / s, z, bits, clip)
        codes[:, col] = c
        d = W[:, col] - s * (c - z)               # w_q - quant(w_q)
        idx = np.array(free)
        k = free.index(col)
        hq = Hinv[np.ix_(idx, [col])][:, 0]      # (H_F^{-1})_{F,q}
        W[:, idx] -= np.outer(d / Hinv[col, col], hq)
        # downdate: H_F^{-1} <- H_F^{-1} - H_F^{-1} e_q e_q^T H_F^{-1} / (H_F^{-1})_qq
        Hinv[np.ix_(idx, idx)] -= np.outer(hq, hq) / Hinv[col, col]
        free.pop(k)
    return codes


def gptq(H, W_hat, scale, zero, bits, group, order=None, clip=True, hint=None, tol=1e-4, R=None,
         return_E=False):
    """The compensation route through R (see the module docstring).

    order: processing order of the original columns (None = natural).  The factor R
    belongs to the reordered curvature H[order][:, order]; pass it to skip the
    factorisation.  hint: codes [d_o x d_i] (original positions) used only at
    near-boundary elements (oracle.grid.round_codes).  Returns (codes, adoptions)
    and, with return_E, the scaled errors E [d_o x d_i] in processing order."""
    W_hat = np.asarray(W_hat, np.float64)
    d_o, d_i = W_hat.shape
    order = np.arange(d_i) if order is None else np.asarray(order)
    if R is None:
        Hp = np.asarray(H, np.float64)[np.ix_(order, order)]
        R = inverse_factor(Hp)
    Wp = W_hat[:, order]
    codes = np.zeros((d_o, d_i), np.int64)
    E = np.zeros((d_o, d_i), order="F")        # scaled errors, processing order
    adopted = 0
    for k in range(d_i):
        col = order[k]
        w = Wp[:, k] - E[:, :k] @ R[:k, k]     # every earlier column's compensation
        s, z = _column_grid(scale, zero, group, col)
        h = None if hint is None else hint[:, col]
        c, n, _ = round_codes(w / s, z, bits, clip, h, tol)
        adopted += n
        codes[:, col] = c
        E[:, k] = (w - s * (c - z)) / R[k, k]
    if return_E:
        return codes, adopted, np.ascontiguousarray(E)
    return codes, adopted
