"""Lattice view of one row: nearest-plane rounding, exhaustive search, error bound.
TEST INFRASTRUCTURE ONLY.

Babai page, technical summary:
* 2.1 -- quantizing one row is a closest-vector problem: lattice basis X diag(s),
  target X w; Theorem 1: any factorisation of X^T X gives an equivalent instance,
  so a square Cholesky factor can stand in for the tall X.
* 2.2 -- Theorem 4: GPTQ run from the last column to the first is Babai's
  nearest-plane algorithm without LLL reduction; applying GPTQ-style propagation
  after Babai changes nothing.
* 2.3 -- Theorem 5: without clipping the error of one row is at most
  (1/4) (T^{-1} s)^T D (T^{-1} s), D the diagonal of the LDL factorisation of the
  reordered Hessian, T the permutation of the quantization order.

Working in code units: with per-column scale s_j and zero z_j a row is
v_j = w_j / s_j + z_j, an integer vector c gives the row w - q = S (v - c), and the
row error is (v - c)^T (S H S) (v - c).
"""
from __future__ import annotations

import itertools

import numpy as np


def code_units(w, s, z):
    return np.asarray(w, np.float64) / s + z


def babai_upper(G_upper: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Nearest plane with an upper-triangular basis G (Gram = G^T G), processing
    coordinates from the last to the first:
        c_k = rint(v_k + sum_{j>k} (G_kj / G_kk) (v_j - c_j)),
    i.e. c_k minimises |(G (v - c))_k| given the later coordinates.  No clipping."""
    d = v.shape[0]
    c = np.zeros(d)
    for k in range(d - 1, -1, -1):
        acc = v[k] + np.dot(G_upper[k, k + 1:] / G_upper[k, k], v[k + 1:] - c[k + 1:])
        c[k] = np.rint(acc)
    return c.astype(np.int64)


def babai_row_cholesky(H, w, s, z):
    """Babai on one row with the Cholesky factor of the scaled Gram S H S."""
    S = np.diag(np.asarray(s, np.float64))
    Gs = S @ np.asarray(H, np.float64) @ S
    G = np.linalg.cholesky(Gs).T                 # upper, Gs = G^T G
    return babai_upper(G, code_units(w, s, z))


def babai_row_qr(X, w, s, z):
    """Babai on one row with the tall basis X diag(s) reduced by QR (Theorem 1:
    the R factor of X diag(s) is, up to signs, the Cholesky factor of its Gram)."""
    B = np.asarray(X, np.float64) * np.asarray(s, np.float64)[None, :]
    _, Rq = np.linalg.qr(B)
    sign = np.sign(np.diag(Rq))
    Rq = Rq * sign[:, None]
    return babai_upper(Rq, code_units(w, s, z))


def ldl_diagonal(H: np.ndarray) -> np.ndarray:
    """Diagonal D of H = L D L^T (L unit lower triangular), by plain elimination."""
    A = np.array(H, np.float64)
    d = A.shape[0]
    D = np.zeros(d)
    for k in range(d):
        D[k] = A[k, k]
        if k + 1 < d:
            l = A[k + 1:, k] / D[k]
            A[k + 1:, k + 1:] -= np.outer(l, A[k, k + 1:])
    return D


def theorem5_bound(H, s, order):
    """Per-row bound on (w - q)^T H (w - q) without clipping when columns are
    quantized in `order`: (1/4) sum_k D_k s_{order'(k)}^2, where D is the LDL
    diagonal of H reordered so that the column quantized LAST is eliminated first
    (the nearest-plane recursion eliminates in the reverse of the quantization order)."""
    order = np.asarray(order)
    elim = order[::-1]
    D = ldl_diagonal(np.asarray(H, np.float64)[np.ix_(elim, elim)])
    s = np.asarray(s, np.float64)
    return 0.25 * float(np.sum(D * s[elim] ** 2))


def enumerate_row(H, w, s, z, bits):
    """Exhaustive minimum of (w - q)^T H (w - q) over every code vector in
    {0 .. 2^b - 1}^d on the fixed grid (s, z).  Returns (best codes, best value)."""
    H = np.asarray(H, np.float64)
    w = np.asarray(w, np.float64)
    s = np.asarray(s, np.float64)
    z = np.asarray(z, np.float64)
    d = w.shape[0]
    levels = np.arange(1 << bits, dtype=np.float64)
    best_v, best_c = np.inf, None
    # iterate the last coordinates in a vectorised block, the rest in Python
    nv = min(d, 4)
    tail = np.array(list(itertools.product(levels, repeat=nv)))       # [L^nv x nv]
    for head in itertools.product(levels, repeat=d - nv):
        c = np.concatenate([np.broadcast_to(np.array(head), (tail.shape[0], d - nv)), tail], axis=1)
        e = w[None, :] - s[None, :] * (c - z[None, :])
        val = np.einsum("ki,ij,kj->k", e, H, e)
        i = int(np.argmin(val))
        if val[i] < best_v:
            best_v, best_c = float(val[i]), c[i].astype(np.int64)
    return best_c, best_v
