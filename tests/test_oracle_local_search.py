"""Pins of the local-search oracle (CPU only): the move-change formula against direct
recomputation of the objective, the vectorised best move against the literal
enumeration, exactness and monotonicity of a step, the conflict-free accept rule, and
that a converged row is a local optimum for every single and pair move."""
import numpy as np
import pytest

from oracle import grid, local_search as ls, objective


def _row_problem(seed, d_i=16, group=8, bits=3, n=60):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((n, d_i))
    A[:, 3] = A[:, 2] * 0.9 + 0.1 * A[:, 3]        # correlated channels
    H = A.T @ A + 0.05 * np.eye(d_i)
    w = (rng.standard_normal(d_i) * 0.3).astype(np.float32)
    s, z = grid.fit_grid_f32(w[None, :], bits, group)
    c = grid.rtn_f32(w[None, :], s, z, bits, group)[0].astype(np.int64)
    return H, w, c, s[0], z[0]


def _f(H, w, c, s, z, group):
    q = grid.dequant(c[None, :], s[None, :], z[None, :], group)
    return float(objective.row_objective(H, w[None, :], q)[0])


def test_move_change_formula_by_recomputation():
    H, w, c, s, z = _row_problem(1)
    group, maxq = 8, 7
    q = grid.dequant(c[None, :], s[None, :], z[None, :], group)[0]
    g = H @ (q - w.astype(np.float64))
    f0 = _f(H, w, c, s, z, group)
    for gi in range(2):
        sl = slice(gi * group, (gi + 1) * group)
        f, j, k, a, b = ls._candidates(g[sl], H[sl, sl], np.diag(H)[sl], c[sl], float(s[gi]), maxq)
        assert len(f) > 0
        for t in range(len(f)):
            c2 = c.copy()
            c2[gi * group + j[t]] += a[t]
            if k[t] != j[t]:
                c2[gi * group + k[t]] += b[t]
            assert abs((_f(H, w, c2, s, z, group) - f0) - f[t]) <= 1e-10 * max(1.0, abs(f0))


@pytest.mark.parametrize("seed", range(8))
def test_best_move_is_the_canonical_minimum(seed):
    rng = np.random.default_rng(100 + seed)
    n, maxq = 12, 3
    A = rng.standard_normal((30, n))
    Hb = A.T @ A
    g = rng.standard_normal(n) * 3
    codes = rng.integers(0, maxq + 1, n)           # includes clipped coordinates
    s = 0.25
    if seed == 0:
        g[:] = 0.0                                  # ties everywhere: tie-break decides
        Hb = -np.ones((n, n)) + 2 * n * np.eye(n)
    f, j, k, a, b = ls._candidates(g, Hb, np.diag(Hb), codes, s, maxq)
    o = np.lexsort((b, a, k, j, f))[0]
    got = ls.best_move(g, Hb, np.diag(Hb), codes, s, maxq)
    if f[o] < 0:
        assert got is not None
        assert got[1:] == (j[o], k[o], a[o], b[o])
        assert abs(got[0] - f[o]) <= 1e-12 * abs(f[o])
    else:
        assert got is None


@pytest.mark.parametrize("seed", range(5))
def test_step_lowers_f_by_the_accepted_running_values(seed):
    H, w, c, s, z = _row_problem(10 + seed, d_i=24, group=8, bits=2)
    f0 = _f(H, w, c, s, z, 8)
    new, acc, _ = ls.step_row(H, w, c, s, z, 2, 8)
    f1 = _f(H, w, new, s, z, 8)
    if acc:
        assert f1 < f0
    assert abs((f1 - f0) - sum(r for _, _, r in acc)) <= 1e-10 * max(1.0, f0)
    assert all(r < 0 for _, _, r in acc)
    assert np.all((new >= 0) & (new <= 3))


def test_conflicting_proposals_accept_only_the_first():
    # two groups, one coordinate each that wants to move up; a strong positive coupling
    # makes the pair of moves worse than either alone
    H = np.array([[1.0, 0.99], [0.99, 1.0]])
    s = np.array([1.0, 1.0], np.float32)
    z = np.array([0, 0], np.uint8)
    w = np.array([0.55, 0.55], np.float32)
    c = np.array([0, 0])
    new, acc, _ = ls.step_row(H, w, c, s, z, 2, 1)
    assert [gi for gi, _, _ in acc] == [0]
    assert list(new) == [1, 0]
    # each move alone lowers f; together they would raise it
    f = lambda cc: _f(H, w, np.array(cc), s, z, 1)
    assert f([1, 0]) < f([0, 0]) and f([0, 1]) < f([0, 0]) and f([1, 1]) > f([1, 0])


def test_converged_row_is_a_local_optimum():
    H, w, c, s, z = _row_problem(3, d_i=16, group=8, bits=3)
    out = ls.local_search(H, w[None, :], c[None, :], s[None, :], z[None, :], 3, 8, 200)
    cf = out["codes"][0]
    assert out["steps"][0] < 200
    f0 = _f(H, w, cf, s, z, 8)
    assert f0 <= _f(H, w, c, s, z, 8)
    for gi in range(2):
        for j in range(8):
            for k in range(j, 8):
                for a in (-1, 1):
                    for b in ((a,) if k == j else (-1, 1)):
                        c2 = cf.copy()
                        c2[gi * 8 + j] += a
                        if k != j:
                            c2[gi * 8 + k] += b
                        if np.any(c2 < 0) or np.any(c2 > 7):
                            continue
                        assert _f(H, w, c2, s, z, 8) >= f0 - 1e-12


def test_on_grid_weights_make_no_move():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((40, 8))
    H = A.T @ A
    s = np.array([0.5], np.float32)
    z = np.array([2], np.uint8)
    c = rng.integers(0, 8, 8)
    w = (s[0] * (c - 2.0)).astype(np.float32)
    out = ls.local_search(H, w[None, :], c[None, :], s[None, :], z[None, :], 3, 8, 5)
    assert out["moves"].sum() == 0
    np.testing.assert_array_equal(out["codes"][0], c)


def test_hints_are_adopted_only_within_the_tolerance():
    H, w, c, s, z = _row_problem(7, d_i=16, group=8, bits=3)
    new, acc, ad = ls.step_row(H, w, c, s, z, 3, 8)
    assert acc
    same, _, ad0 = ls.step_row(H, w, c, s, z, 3, 8, hint=new, tol=1e-9)
    np.testing.assert_array_equal(same, new)
    assert ad0 == 0
    # a hint that leaves out the first accepted move: adopted only if that move's running
    # value is within the tolerance of zero
    gi, m, run = acc[0]
    alt = new.copy()
    alt[gi * 8 + m[1]] -= m[3]
    if m[2] != m[1]:
        alt[gi * 8 + m[2]] -= m[4]
    strict, _, _ = ls.step_row(H, w, c, s, z, 3, 8, hint=alt, tol=1e-12)
    assert not np.array_equal(strict, alt)
    loose, _, ad2 = ls.step_row(H, w, c, s, z, 3, 8, hint=alt, tol=abs(run) * 1.01)
    assert ad2 >= 1
    assert loose[gi * 8 + m[1]] == c[gi * 8 + m[1]]
