"""Pins of the order oracle (CPU only): act order and min-pivot order against hand-derived
cases, the min-pivot rule against Schur complements computed by linear solves, the
invariant product of pivots, the diagonal special case, and the per-layer bound against
Theorem 5 on no-clip GPTQ results."""
import numpy as np
import pytest

from oracle import gptq, grid, lattice, objective, order


def _spd(rng, d, n=None):
    n = 3 * d if n is None else n
    X = rng.standard_normal((n, d)) * rng.uniform(0.2, 5.0, d)
    X[:, 1] = X[:, 0] * 0.8 + 0.2 * X[:, 1]
    return X.T @ X + 1e-2 * np.eye(d)


def test_act_order_hand_case():
    H = np.diag([3.0, 5.0, 5.0, 1.0])
    np.testing.assert_array_equal(order.act_order(H), [1, 2, 0, 3])


def test_min_pivot_hand_cases():
    # equal diagonals: the larger index is eliminated first (quantized last); second
    # pivot 2 - 1/2
    perm, D, _ = order.min_pivot_order(np.array([[2.0, 1.0], [1.0, 2.0]]))
    np.testing.assert_array_equal(perm, [0, 1])
    np.testing.assert_allclose(D, [1.5, 2.0], rtol=0, atol=1e-15)
    # the Schur update changes the order: eliminate 1 (diag 1), then 0 (4 - 1.9^2 = 0.39),
    # then 2 (2); act order would quantize 0, 2, 1
    H = np.array([[4.0, 1.9, 0.0], [1.9, 1.0, 0.0], [0.0, 0.0, 2.0]])
    perm, D, _ = order.min_pivot_order(H)
    np.testing.assert_array_equal(perm, [2, 0, 1])
    np.testing.assert_allclose(D, [2.0, 0.39, 1.0], rtol=1e-14)
    np.testing.assert_array_equal(order.act_order(H), [0, 2, 1])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_min_pivot_is_smallest_schur_diagonal_at_every_step(seed):
    rng = np.random.default_rng(seed)
    d = 12
    H = _spd(rng, d)
    perm, D, _ = order.min_pivot_order(H)
    elim = list(perm[::-1])
    piv = D[::-1]
    for t in range(d):
        done = elim[:t]
        rest = [j for j in range(d) if j not in done]
        sd = np.array([order.schur_diagonal(H, done, j) for j in rest])
        chosen = order.schur_diagonal(H, done, elim[t])
        assert abs(chosen - piv[t]) <= 1e-9 * H[elim[t], elim[t]]
        assert np.all(chosen <= sd + 1e-9 * np.max(np.diag(H)))


@pytest.mark.parametrize("seed", [4, 5])
def test_pivots_match_ldl_of_reordered_matrix_and_determinant(seed):
    rng = np.random.default_rng(seed)
    H = _spd(rng, 20)
    perm, D, _ = order.min_pivot_order(H)
    np.testing.assert_allclose(D, order.pivots_for_order(H, perm), rtol=1e-10)
    sign, logdet = np.linalg.slogdet(H)
    assert sign > 0
    assert abs(np.sum(np.log(D)) - logdet) <= 1e-9 * abs(logdet) + 1e-9
    # a permutation of 0..d-1
    np.testing.assert_array_equal(np.sort(perm), np.arange(20))


def test_diagonal_hessian_min_pivot_is_act_order():
    rng = np.random.default_rng(6)
    dg = rng.uniform(0.5, 3.0, 15)
    dg[4] = dg[9]          # a tie
    H = np.diag(dg)
    perm, D, _ = order.min_pivot_order(H)
    np.testing.assert_array_equal(perm, order.act_order(H))
    np.testing.assert_allclose(D, dg[perm], rtol=0)


def test_layer_bound_is_theorem5_with_half_factor():
    rng = np.random.default_rng(7)
    d, group, rows = 16, 4, 3
    H = _spd(rng, d)
    s = rng.uniform(0.005, 0.03, (rows, d // group)).astype(np.float32)
    perm = rng.permutation(d)
    b = order.layer_bound(H, s, group, perm)
    for r in range(rows):
        s_col = np.repeat(s[r], group)
        assert abs(b[r] - 0.5 * lattice.theorem5_bound(H, s_col, perm)) <= 1e-12 * b[r]


@pytest.mark.parametrize("which", ["natural", "act", "min_pivot"])
def test_no_clip_gptq_objective_within_bound(which):
    rng = np.random.default_rng(8)
    worst = 0.0
    for _ in range(20):
        d, group, rows = 24, 8, 4
        H = _spd(rng, d)
        W = (rng.standard_normal((rows, d)) * 0.05).astype(np.float32)
        s, z = grid.fit_grid_f32(W, 2, group)
        perm = {"natural": np.arange(d), "act": order.act_order(H),
                "min_pivot": order.min_pivot_order(H)[0]}[which]
        codes, _ = gptq.gptq(H, W, s, z, 2, group, order=perm, clip=False)
        f = objective.row_objective(H, W, grid.dequant(codes, s, z, group))
        b = order.layer_bound(H, s, group, perm)
        assert np.all(f <= b * (1 + 1e-9))
        worst = max(worst, float(np.max(f / b)))
    assert worst > 0.1          # not vacuous


def test_hint_adoption_only_within_tolerance():
    H = np.diag([1.0, 1.0 + 1e-13, 3.0])
    perm, D, ad = order.min_pivot_order(H)
    np.testing.assert_array_equal(perm, [2, 1, 0])
    assert ad == 0
    # a hint that eliminates 1 first (within 1e-12 of the smallest): adopted
    perm2, _, ad2 = order.min_pivot_order(H, hint=np.array([2, 0, 1]), tol=1e-12)
    np.testing.assert_array_equal(perm2, [2, 0, 1])
    assert ad2 == 1
    # outside the tolerance: not adopted
    perm3, _, ad3 = order.min_pivot_order(H, hint=np.array([2, 0, 1]), tol=1e-14)
    np.testing.assert_array_equal(perm3, [2, 1, 0])
    assert ad3 == 0
    # a hint equal to the result is never counted
    assert order.min_pivot_order(H, hint=perm, tol=1.0)[2] == 0
