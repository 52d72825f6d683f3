"""Pairwise-swap local search on the grid.  TEST INFRASTRUCTURE ONLY.

ADMM-Q summary, methodology, 2. key algorithmic components, the local-search item: a
post-processing step that evaluates discrete moves which directly lower the
reconstruction error, swapping values between rows (input channels in the page's
d_i x d_o layout, i.e. coordinates of one output channel here), run in parallel.

The pages give no move set, order or acceptance rule; this module fixes them (the
plainest reading, shared with the library):

* State: codes C of one output row on a fixed grid (s, z per group); the error
  e = q - w_hat with q = s (C - z); the objective f = 1/2 e^T H e; its gradient g = H e.
* Moves inside one group (one scale s): a single move changes one code by a = +-1;
  a pair move (the swap) changes codes j < k by a, b in {-1, +1} (a = -b moves one grid
  step from one coordinate to the other).  Codes stay in [0, 2^bits - 1].  With
  d_j = a s, d_k = b s the exact change of f is
      single:  d_j g_j + 1/2 d_j^2 H_jj
      pair:    d_j g_j + d_k g_k + 1/2 (d_j^2 H_jj + d_k^2 H_kk) + d_j d_k H_jk.
* One step: every group proposes its best move (smallest change; ties to the smallest
  (j, k, a, b) with singles written k = j, b = a, and -1 before +1), if that change is
  negative.  Proposals are accepted group by group in ascending order: a proposal is
  accepted when its change plus its exact interaction with the moves already accepted
  this step, sum over p in it, p' in them of d_p d_p' H_pp', is still negative.  The
  accepted moves are applied together, so f decreases by exactly the sum of those
  running values.  Rows are independent.  A row stops when a step accepts nothing.
"""
from __future__ import annotations

import numpy as np

from .grid import dequant


def _candidates(g, Hb, Hd, codes, s, maxq):
    """All moves of one group: returns (delta_f [m], j [m], k [m], a [m], b [m]) in the
    canonical order (j, k, a, b) ascending with singles as k = j."""
    n = len(g)
    out_f, out_j, out_k, out_a, out_b = [], [], [], [], []
    for j in range(n):
        for k in range(j, n):
            for a in (-1, 1):
                for b in ((a,) if k == j else (-1, 1)):
                    if not (0 <= codes[j] + a <= maxq):
                        continue
                    if k != j and not (0 <= codes[k] + b <= maxq):
                        continue
                    dj = a * s
                    if k == j:
                        df = dj * g[j] + 0.5 * dj * dj * Hd[j]
                    else:
                        dk = b * s
                        df = (dj * g[j] + dk * g[k] + 0.5 * (dj * dj * Hd[j] + dk * dk * Hd[k])
                              + dj * dk * Hb[j, k])
                    out_f.append(df)
                    out_j.append(j)
                    out_k.append(k)
                    out_a.append(a)
                    out_b.append(b)
    return (np.array(out_f), np.array(out_j), np.array(out_k), np.array(out_a),
            np.array(out_b))


def best_move(g, Hb, Hd, codes, s, maxq):
    """Best move of one group as (delta_f, j, k, a, b), or None if no move lowers f.
    The same candidates and order as _candidates, evaluated as arrays."""
    n = len(g)
    c = np.asarray(codes, np.int64)
    u = {}
    for a in (-1, 1):
        ok = (c + a >= 0) & (c + a <= maxq)
        u[a] = np.where(ok, a * s * g + 0.5 * s * s * Hd, np.inf)
    iu = np.triu_indices(n, 1)
    vals, js, ks, As, Bs = [], [], [], [], []
    for a in (-1, 1):
        vals.append(u[a]); js.append(np.arange(n)); ks.append(np.arange(n))
        As.append(np.full(n, a)); Bs.append(np.full(n, a))
    for a in (-1, 1):
        for b in (-1, 1):
            M = u[a][:, None] + u[b][None, :] + a * b * s * s * Hb
            vals.append(M[iu]); js.append(iu[0]); ks.append(iu[1])
            As.append(np.full(len(iu[0]), a)); Bs.append(np.full(len(iu[0]), b))
    v = np.concatenate(vals)
    if not np.any(np.isfinite(v)):
        return None
    m = np.min(v)
    if not m < 0:
        return None
    sel = np.nonzero(v == m)[0]
    j, k, aa, bb = (np.concatenate(x)[sel] for x in (js, ks, As, Bs))
    o = np.lexsort((bb, aa, k, j))[0]
    return (float(m), int(j[o]), int(k[o]), int(aa[o]), int(bb[o]))


def _cross(m1, m2, s1, s2, H, c1, c2):
    """Interaction d^T H d' of two moves in different groups (column offsets c1, c2)."""
    p1 = [(c1 + m1[1], m1[3] * s1)] + ([(c1 + m1[2], m1[4] * s1)] if m1[2] != m1[1] else [])
    p2 = [(c2 + m2[1], m2[3] * s2)] + ([(c2 + m2[2], m2[4] * s2)] if m2[2] != m2[1] else [])
    return sum(dp * dq * H[p, q] for p, dp in p1 for q, dq in p2)


def step_row(H, w, codes, scale, zero, bits, group, hint=None, tol=0.0):
    """One step on one row.  hint: the codes the other side produced for this step; at a
    decision whose margin is within tol (a proposal within tol of the best, or a running
    value within tol of zero) the hint's choice is adopted.  Returns (new codes, accepted
    [(group, move, running value)], adoptions)."""
    H = np.asarray(H, np.float64)
    codes = np.asarray(codes, np.int64)
    maxq = (1 << bits) - 1
    q = dequant(codes[None, :], scale[None, :], zero[None, :], group)[0]
    e = q - np.asarray(w, np.float64)
    g = H @ e
    G = len(codes) // group
    accepted = []
    adopted = 0
    new = codes.copy()
    for gi in range(G):
        c0 = gi * group
        sl = slice(c0, c0 + group)
        s = float(scale[gi])
        Hb = H[sl, sl]
        Hd = np.diag(Hb)
        mine = best_move(g[sl], Hb, Hd, codes[sl], s, maxq)
        theirs = None
        if hint is not None:
            diff = np.nonzero(np.asarray(hint[sl], np.int64) != codes[sl])[0]
            if len(diff):
                j = int(diff[0])
                k = int(diff[-1])
                a = int(hint[c0 + j] - codes[c0 + j])
                b = int(hint[c0 + k] - codes[c0 + k])
                dj, dk = a * s, b * s
                if k == j:
                    df = dj * g[c0 + j] + 0.5 * dj * dj * Hd[j]
                else:
                    df = (dj * g[c0 + j] + dk * g[c0 + k] + 0.5 * (dj * dj * Hd[j] + dk * dk * Hd[k])
                          + dj * dk * Hb[j, k])
                theirs = (df, j, k, a, b)
        prop = mine
        if hint is not None and theirs != mine:
            if theirs is not None and (mine is None or theirs[0] <= mine[0] + tol):
                prop = theirs
                adopted += int(mine is None or theirs[1:] != mine[1:])
            elif theirs is None and mine is not None:
                prop = mine    # decided by the running value below
        if prop is None:
            continue
        run = prop[0] + sum(_cross(prop, m, s, float(scale[g2]), H, c0, g2 * group)
                            for g2, m, _ in accepted)
        take = run < 0
        if hint is not None:
            hinted = theirs is not None and tuple(prop[1:]) == tuple(theirs[1:])
            if take != hinted and abs(run) <= tol:
                take = hinted
                adopted += 1
        if take:
            accepted.append((gi, prop, run))
    for gi, m, _ in accepted:
        c0 = gi * group
        new[c0 + m[1]] += m[3]
        if m[2] != m[1]:
            new[c0 + m[2]] += m[4]
    return new, accepted, adopted


def local_search(H, W_hat, codes, scale, zero, bits, group, max_steps, hints=None, tol=0.0):
    """Rows of W_hat [rows x d_i] from codes [rows x d_i] on the fixed grid; at most
    max_steps steps per row.  hints[t] (optional) are the other side's codes after step
    t.  Returns dict(codes, steps [rows], moves [max_steps] (accepted moves summed over
    the rows), adopted)."""
    codes = np.array(codes, np.int64)
    rows = codes.shape[0]
    moves = np.zeros(max_steps, np.int64)
    steps = np.zeros(rows, np.int64)
    adopted = 0
    for r in range(rows):
        for t in range(max_steps):
            h = None if hints is None else hints[t][r]
            new, acc, ad = step_row(H, W_hat[r], codes[r], scale[r], zero[r], bits, group, h, tol)
            adopted += ad
            if not acc:
                break
            codes[r] = new
            moves[t] += len(acc)
            steps[r] = t + 1
    return dict(codes=codes, steps=steps, moves=moves, adopted=adopted)
