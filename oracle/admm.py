"""ADMM-Q.  TEST INFRASTRUCTURE ONLY.

ADMM-Q page, technical summary, 2. key algorithmic components:

* diagonal scaling Sigma = Diag(H)^(-1/2) -- read as the change of variables
  W~ = W Sigma^{-1} (column j multiplied by sqrt(H_jj)), so the objective becomes
  (1/2) Tr((W~ - W~_hat) H~ (W~ - W~_hat)^T) with H~ = Sigma H Sigma (unit diagonal);
* ADMM splitting with an auxiliary D (the quantized copy):
  1. W-update: the continuous minimiser of the objective plus the penalty
     (rho/2)||W~ - (D~ - U)||^2, i.e. W~ = (W~_hat H~ + rho M)(H~ + rho I)^{-1} with
     M = D~ - U, evaluated through the eigendecomposition H~ = V Lambda V^T as
     W~ = ((P + rho M V) / (Lambda + rho)) V^T with P = W~_hat V Lambda;
  2. D-update: projection onto the grid, which in original coordinates is plain
     round-to-nearest with clipping (the penalty weights every element by H_jj,
     which does not move the nearest point of a one-dimensional grid);
  3. dual update of the Lagrange multiplier;
* grid refresh: scale and zero refit from the current continuous iterate;
* penalty schedule rho_t = rho_0 gamma^t, under which the continuous and the discrete
  iterates reach the same limit.

Readings where the pages are silent (all selectable, defaults first):
* dual: the multiplier Y = rho U is kept across a change of rho, so after
  U += W~ - D~ the scaled dual is rescaled by rho_t / rho_{t+1} ("lagrange");
  "scaled" keeps U += W~ - D~ alone.
* refresh: per (row, group), min/max of the continuous iterate W = W~ Sigma, forced to
  hold 0, then clamped into the group's initial range [lo_0, hi_0] so a refresh can only
  narrow the grid ("clamped"); "unclamped" takes the fit as is; "from_z" fits W + U Sigma.
  A range the clamp closes to a point (hi = lo = 0) defines no grid: the group keeps
  its current scale and zero.
* refresh at iterations t with t mod k == 0 (k = refresh_every; 0 = never).
* start: D^0 = RTN(W_hat) on the static fp32 grid of W_hat, U^0 = 0; t runs t0 .. t0+T-1.
* output: the last discrete iterate and its grid.
* residuals: r_p = ||W~ - D~^{t+1}||_F and r_d = rho_t ||D~^{t+1} - D~^t||_F (scaled space).

Pins: the whole loop against a trajectory derived by hand in exact rational
arithmetic (tests/golden/admm_trajectory.json: three iterations with the refresh,
the clamp, the dual rescale and the rho_t indexing all visible); the W-update against
the linear-solve definition; T = 0 and rho_0 -> infinity reduce to RTN; on-grid inputs
are fixed points; exhaustive enumeration bounds the result from below; the primal
residual vanishes under the rho schedule.  The pages print no ADMM-Q numbers, so the
readings themselves (listed above) are the pages' plainest reading, not pinned values.
"""
from __future__ import annotations

import numpy as np

from .grid import (F32, dequant, fit_range_f32, fit_range_f64, grid_from_range_f32,
                   grid_from_range_f64, round_codes, rtn_f32)


def spectral(H: np.ndarray):
    """Sigma (vector), H~ = Sigma H Sigma, and its eigendecomposition (Lambda, V)."""
    H = np.asarray(H, np.float64)
    sig = 1.0 / np.sqrt(np.diag(H))
    Ht = H * sig[:, None] * sig[None, :]
    lam, V = np.linalg.eigh(Ht)
    return sig, Ht, lam, V


def w_update_eig(P, M, V, lam, rho):
    """W~ = ((P + rho M V) diag(1 / (Lambda + rho))) V^T."""
    return ((P + rho * (M @ V)) / (lam + rho)[None, :]) @ V.T


def w_update_solve(Ht, Wt_hat, M, rho, WtH=None):
    """The definition: W~ (H~ + rho I) = W~_hat H~ + rho M, solved directly (the matrix
    is symmetric positive definite: Cholesky).  WtH: W~_hat H~ if already formed."""
    from scipy.linalg import cho_factor, cho_solve
    A = np.array(Ht, np.float64)
    A[np.diag_indices_from(A)] += rho
    rhs = (Wt_hat @ Ht if WtH is None else WtH) + rho * M
    return cho_solve(cho_factor(A, lower=True, overwrite_a=True, check_finite=False), rhs.T,
                     check_finite=False).T


def initial_grid(W_hat_f32: np.ndarray, bits: int, group: int):
    """Static fp32 grid of W_hat, its range (lo_0, hi_0) and D^0 = RTN(W_hat)."""
    lo0, hi0 = fit_range_f32(W_hat_f32, group)
    s0, z0 = grid_from_range_f32(lo0, hi0, bits)
    c0 = rtn_f32(W_hat_f32, s0, z0, bits, group)
    return lo0, hi0, s0, z0, c0


def admm(H, W_hat_f32, bits, group, iters, rho0, gamma, refresh_every=1, *,
         refresh="clamped", dual="lagrange", state=None, hints=None, zero_hints=None,
         tol=1e-4, spec=None, trace=False, wupdate="eig"):
    """Run ADMM-Q on the rows of W_hat (fp32 [rows x d_i]; rows are independent, so any
    subset of a layer's rows can be run on its own).

    state: warm start dict(t0, codes, scale, zero, U) from an earlier call.
    hints / zero_hints: per-iteration codes [rows x d_i] / zero points [rows x G]
      (indexed by t - t0), used only at near-boundary elements.
    wupdate: "eig" (the eigendecomposition form) or "solve" (a Cholesky solve of
      (H~ + rho_t I) per iteration; no eigendecomposition, for short runs on large H).
      spec: (sigma, H~, Lambda, V) if already computed ("solve" uses sigma and H~ only).
    Returns dict(codes, scale, zero, U, res [iters x 2], adopted, trace)."""
    W_hat_f32 = np.asarray(W_hat_f32, F32)
    rows, d_i = W_hat_f32.shape
    if wupdate == "eig":
        sig, Ht, lam, V = spec if spec is not None else spectral(H)
    elif wupdate == "solve":
        if spec is not None:
            sig, Ht = spec[0], spec[1]
        else:
            Hd = np.asarray(H, np.float64)
            sig = 1.0 / np.sqrt(np.diag(Hd))
            Ht = Hd * sig[:, None] * sig[None, :]
    else:
        raise ValueError(f"unknown wupdate {wupdate!r}")
    Wt_hat = W_hat_f32.astype(np.float64) / sig[None, :]
    if wupdate == "eig":
        P = (Wt_hat @ V) * lam[None, :]
    else:
        WtH = Wt_hat @ Ht
    lo0, hi0, s0, z0, c0 = initial_grid(W_hat_f32, bits, group)
    if state is None:
        t0, C, scale, zero, U = 0, c0.astype(np.int64), s0, z0.astype(np.int64), np.zeros((rows, d_i))
    else:
        t0 = int(state["t0"])
        C = np.asarray(state["codes"], np.int64)
        scale = np.asarray(state["scale"], F32)
        zero = np.asarray(state["zero"], np.int64)
        U = np.asarray(state["U"], np.float64).copy()
    res = np.zeros((iters, 2))
    adopted = 0
    tr = []
    for k in range(iters):
        t = t0 + k
        rho = rho0 * gamma ** t
        rho_next = rho0 * gamma ** (t + 1)
        Dt = dequant(C, scale, zero, group) / sig[None, :]
        M = Dt - U
        if wupdate == "eig":
            Wt = w_update_eig(P, M, V, lam, rho)
        else:
            Wt = w_update_solve(Ht, Wt_hat, M, rho, WtH)
        if refresh_every > 0 and t % refresh_every == 0 and refresh != "off":
            src = (Wt + U) * sig[None, :] if refresh == "from_z" else Wt * sig[None, :]
            lo, hi = fit_range_f64(src, group)
            if refresh in ("clamped", "from_z"):
                lo = np.maximum(lo, lo0.astype(np.float64))
                hi = np.minimum(hi, hi0.astype(np.float64))
            # after the clamp the range can close (hi == lo == 0: a group whose initial
            # range starts at 0 while the iterate lies entirely on the other side); no
            # grid has that range, so such a group keeps the grid it had
            keep = hi <= lo
            zh = None if zero_hints is None else zero_hints[k]
            # (a stand-in range [-1, 2] for those groups keeps the division finite and its
            # zero point, (2^b - 1)/3, away from a rounding boundary; it is discarded)
            s_new, z_new, n = grid_from_range_f64(np.where(keep, -1.0, lo),
                                                  np.where(keep, 2.0, hi), bits, zh, tol)
            scale = np.where(keep, scale, s_new).astype(F32)
            zero = np.where(keep, zero, z_new).astype(np.int64)
            adopted += n
        s_full = np.repeat(scale.astype(np.float64), group, axis=1)
        z_full = np.repeat(zero.astype(np.float64), group, axis=1)
        Z = (Wt + U) * sig[None, :]
        h = None if hints is None else hints[k]
        C_new, n, _ = round_codes(Z / s_full, z_full, bits, True, h, tol)
        adopted += n
        Dt_new = s_full * (C_new - z_full) / sig[None, :]
        U = U + Wt - Dt_new
        if dual == "lagrange":
            U *= rho / rho_next
        res[k, 0] = np.linalg.norm(Wt - Dt_new)
        res[k, 1] = rho * np.linalg.norm(Dt_new - Dt)
        C = C_new
        if trace:
            tr.append((C.copy(), scale.copy(), zero.copy()))
    return dict(codes=C, scale=scale, zero=zero, U=U, res=res, adopted=adopted,
                trace=tr if trace else None, t_end=t0 + iters)
