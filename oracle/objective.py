"""Layer objective.  TEST INFRASTRUCTURE ONLY.

ADMM-Q page, technical summary 1. problem formulation: (1/2) Tr((W - W_hat)^T H (W - W_hat)).
The pages' layout there is W in R^{d_i x d_o}; this package stores weights
[d_o x d_i] (the GPTQ tutorial page's layout, section 2), where the same value is
(1/2) sum over rows r of (w_r - w_hat_r)^T H (w_r - w_hat_r).  The 1/2 matches the
tutorial's worked example (cost 0.04 -> 0.03 for H = [[2,1],[1,2]]).
"""
from __future__ import annotations

import numpy as np


def row_objective(H: np.ndarray, W_hat: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """Per-row (1/2) (w_hat_r - q_r)^T H (w_hat_r - q_r), fp64."""
    D = np.asarray(W_hat, np.float64) - np.asarray(Q, np.float64)
    return 0.5 * np.einsum("rj,rj->r", D @ np.asarray(H, np.float64), D)


def objective(H, W_hat, Q) -> float:
    return float(row_objective(H, W_hat, Q).sum())
