"""Oracle pins for the Hessian, GPTQ, ADMM-Q and the lattice view (CPU only).

Each test ties the oracle to something other than itself: values printed on the
pages (tests/golden), closed forms, textbook reductions, library routines used as an
independent route, brute force on tiny inputs, or invariants that a dropped term,
wrong sign or transposed operand would break."""
import numpy as np
import pytest
import scipy.linalg

import qz_synth
from conftest import golden
from oracle import admm, gptq, grid, hessian, lattice, objective


def spd(d, rng, cond_scale=1.0, n=None):
    n = n or 4 * d
    X = rng.standard_normal((n, d))
    X[:, 0] *= 5 * cond_scale
    X += 0.5 * rng.standard_normal((n, 1))     # correlated channels
    H, _ = hessian.hessian(X, 0.01)
    return X, H


def layer(d_o, d_i, bits, group, rng, sw=0.02):
    W = (rng.standard_normal((d_o, d_i)) * sw).astype(np.float32)
    s, z = grid.fit_grid_f32(W, bits, group)
    return W, s, z


# ------------------------------------------------------------------ Hessian
def test_hessian_matches_triple_loop():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((9, 4)).astype(np.float32)
    G = np.zeros((4, 4))
    for i in range(4):
        for j in range(4):
            for t in range(9):
                G[i, j] += float(X[t, i]) * float(X[t, j])
    H, lam = hessian.hessian(X, 0.01)
    assert lam == pytest.approx(0.01 * np.trace(G) / 4, rel=1e-14)
    np.testing.assert_allclose(H, G + lam * np.eye(4), rtol=1e-14, atol=1e-14)


def test_hessian_bf16_input_and_scaling():
    import qz_synth
    Xb = qz_synth.calib_bf16(7, 300, 24, p_out=0.1, f_out=30.0)
    Xf = qz_synth.bf16_bits_to_f32(Xb)
    H1, _ = hessian.hessian(Xb, 0.01)
    H2, _ = hessian.hessian(Xf, 0.01)
    np.testing.assert_array_equal(H1, H2)
    np.testing.assert_allclose(H1, H1.T, rtol=0, atol=0)
    sig, Ht = hessian.scaling(H1)
    np.testing.assert_allclose(np.diag(Ht), 1.0, rtol=1e-14)
    ii = np.array([0, 3, 23, 5]); jj = np.array([0, 7, 2, 5])
    np.testing.assert_allclose(hessian.gram_entries(Xb, ii, jj), hessian.gram(Xb)[ii, jj],
                               rtol=1e-12)


# ------------------------------------------------------------------ GPTQ worked examples
def test_gptq_worked_example_compensation():
    g = golden("gptq_worked_examples.json")["compensation"]
    H = np.array(g["H"])
    pr = g["printed"]
    # the compensation of the page: delta = d H^{-1} e_q / (H^{-1})_qq
    Hinv = np.linalg.inv(H)
    delta = pr["first_weight_change"] * Hinv[:, 0] / Hinv[0, 0]
    assert delta[1] == pytest.approx(pr["second_weight_change"], abs=1e-15)
    assert 0.5 * np.array([0.2, 0]) @ H @ np.array([0.2, 0]) == pytest.approx(pr["cost_first_only"])
    assert 0.5 * delta @ H @ delta == pytest.approx(pr["cost_compensated"])
    c = g["construction"]
    W = np.array(c["W_hat"], np.float32)
    s = np.array(c["scale"], np.float32); z = np.array(c["zero"], np.uint8)
    rtn = grid.rtn_f32(W, s, z, c["bits"], c["group"])
    np.testing.assert_array_equal(rtn, c["codes_rtn"])
    for route in ("plain", "blocked"):
        if route == "plain":
            codes = gptq.gptq_plain(H, W, s, z, c["bits"], c["group"])
        else:
            codes, _ = gptq.gptq(H, W, s, z, c["bits"], c["group"])
        np.testing.assert_array_equal(codes, c["codes_gptq"])
        q = grid.dequant(codes, s, z, 1)
        assert objective.objective(H, W, q) == pytest.approx(pr["cost_compensated"], rel=1e-6)
        assert q[0, 1] - W[0, 1] == pytest.approx(pr["second_weight_change"], abs=1e-7)
    assert objective.objective(H, W, grid.dequant(rtn, s, z, 1)) == pytest.approx(
        pr["cost_first_only"], rel=1e-6)


def test_gptq_worked_example_collinear_needs_damping():
    g = golden("gptq_worked_examples.json")["collinear"]
    c = g["construction"]
    rng = np.random.default_rng(3)
    x = rng.standard_normal(64)
    X = np.stack([x, x], axis=1)
    G = hessian.gram(X)
    assert np.linalg.matrix_rank(G) == 1            # the curvature is not invertible
    H, lam = hessian.hessian(X, c["damp"])
    W = np.array([g["printed"]["W_hat"]], np.float32)
    s = np.array(c["scale"], np.float32); z = np.array(c["zero"], np.uint8)
    codes, _, E = gptq.gptq(H, W, s, z, c["bits"], c["group"], return_E=True)
    np.testing.assert_array_equal(codes, c["codes_gptq"])
    np.testing.assert_array_equal(gptq.gptq_plain(H, W, s, z, c["bits"], c["group"]), c["codes_gptq"])
    # pre-round value of the second weight: 0.51 + 0.49 / 1.01
    R = gptq.inverse_factor(H)
    pre = float(W[0, 1]) - E[0, 0] * R[0, 1]
    assert pre == pytest.approx(c["second_preround"], rel=1e-6)
    assert grid.dequant(codes, s, z, 1)[0, 0] == g["printed"]["first_quantized"]
    assert grid.dequant(codes, s, z, 1)[0, 1] == g["printed"]["second_target"]


# ------------------------------------------------------------------ GPTQ routes
def test_inverse_factor_lapack_is_the_same_factor():
    # the LAPACK route (potrf, potri, potrf) is the definition's R: upper, positive
    # diagonal, R^T R H = I, and equal to the general-inverse route
    rng = np.random.default_rng(7)
    for d in (1, 9, 64, 131):
        _, H = spd(d, rng, cond_scale=30.0)
        R = gptq.inverse_factor_lapack(H)
        np.testing.assert_array_equal(np.tril(R, -1), 0)
        assert np.all(np.diag(R) > 0)
        np.testing.assert_allclose(R.T @ R @ H, np.eye(d), atol=1e-8)
        np.testing.assert_allclose(R, gptq.inverse_factor(H), rtol=1e-8, atol=1e-10)
    with pytest.raises(np.linalg.LinAlgError):
        gptq.inverse_factor_lapack(-np.eye(3))


def blocked_gptq(H, W_hat, scale, zero, bits, group, B, order=None, clip=True):
    """The tutorial's section 3 evaluation order of the same compensations: blocks of B
    columns; a fixed column's compensation goes at once to the later columns of its own
    block and, for the columns after the block, is collected and applied in one matrix
    product when the block is done.  Written here only to check that the regrouping
    leaves the codes unchanged."""
    d_o, d_i = W_hat.shape
    order = np.arange(d_i) if order is None else np.asarray(order)
    R = gptq.inverse_factor(np.asarray(H, np.float64)[np.ix_(order, order)])
    Wk = np.asarray(W_hat, np.float64)[:, order].copy()
    codes = np.zeros((d_o, d_i), np.int64)
    for a in range(0, d_i, B):
        b = min(a + B, d_i)
        Eb = np.zeros((d_o, b - a))
        for j in range(a, b):
            g = order[j] // group
            sj, zj = np.asarray(scale, np.float64)[:, g], np.asarray(zero, np.float64)[:, g]
            c, _, _ = grid.round_codes(Wk[:, j] / sj, zj, bits, clip)
            codes[:, order[j]] = c
            Eb[:, j - a] = (Wk[:, j] - sj * (c - zj)) / R[j, j]
            Wk[:, j + 1:b] -= np.outer(Eb[:, j - a], R[j, j + 1:b])
        Wk[:, b:] -= Eb @ R[a:b, b:]
    return codes


@pytest.mark.parametrize("clip", [True, False])
def test_gptq_factor_route_equals_lagrange_route(clip):
    rng = np.random.default_rng(11)
    d_i, d_o, bits, group = 40, 12, 3, 8
    _, H = spd(d_i, rng)
    W, s, z = layer(d_o, d_i, bits, group, rng)
    a, _ = gptq.gptq(H, W, s, z, bits, group, clip=clip)
    b = gptq.gptq_plain(H, W, s, z, bits, group, clip=clip)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("B", [1, 3, 16, 40])
@pytest.mark.parametrize("clip", [True, False])
def test_gptq_blocked_evaluation_gives_the_same_codes(B, clip):
    rng = np.random.default_rng(10 + B)
    d_i, d_o, bits, group = 40, 12, 3, 8
    _, H = spd(d_i, rng)
    W, s, z = layer(d_o, d_i, bits, group, rng)
    a, _ = gptq.gptq(H, W, s, z, bits, group, clip=clip)
    np.testing.assert_array_equal(blocked_gptq(H, W, s, z, bits, group, B, clip=clip), a)


def test_gptq_block_size_invariance_and_order():
    rng = np.random.default_rng(5)
    d_i, d_o = 64, 16
    _, H = spd(d_i, rng)
    W, s, z = layer(d_o, d_i, 2, 16, rng)
    ref, _ = gptq.gptq(H, W, s, z, 2, 16)
    for B in (7, 32, 64, 128):
        np.testing.assert_array_equal(blocked_gptq(H, W, s, z, 2, 16, B), ref)
    perm = rng.permutation(d_i)
    a, _ = gptq.gptq(H, W, s, z, 2, 16, order=perm)
    b = gptq.gptq_plain(H, W, s, z, 2, 16, order=perm)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(blocked_gptq(H, W, s, z, 2, 16, 8, order=perm), a)


def test_inverse_factor_is_upper_cholesky_of_inverse():
    rng = np.random.default_rng(6)
    _, H = spd(30, rng)
    R = gptq.inverse_factor(H)
    np.testing.assert_allclose(np.tril(R, -1), 0, atol=0)
    assert np.all(np.diag(R) > 0)
    np.testing.assert_allclose(R.T @ R @ H, np.eye(30), atol=1e-9)
    # reverse-order factorisation: R = (J chol(J H J) J)^{-1}
    J = np.eye(30)[::-1]
    L = np.linalg.cholesky(J @ H @ J)
    np.testing.assert_allclose(np.linalg.inv(J @ L @ J), R, rtol=1e-8, atol=1e-12)


@pytest.mark.parametrize("clip", [True, False])
def test_gptq_objective_is_half_sum_E_squared(clip):
    # per-step cost increase is (1/2) d^2 / (H_F^{-1})_qq = (1/2) E_j^2
    rng = np.random.default_rng(7)
    d_i, d_o = 48, 10
    _, H = spd(d_i, rng)
    W, s, z = layer(d_o, d_i, 3, 16, rng)
    codes, _, E = gptq.gptq(H, W, s, z, 3, 16, clip=clip, return_E=True)
    q = grid.dequant(codes, s, z, 16)
    np.testing.assert_allclose(objective.row_objective(H, W, q), 0.5 * (E ** 2).sum(1), rtol=1e-9)


def test_gptq_diagonal_hessian_is_rtn():
    rng = np.random.default_rng(8)
    H = np.diag(rng.uniform(0.5, 3.0, 32))
    W, s, z = layer(6, 32, 3, 8, rng)
    codes, _ = gptq.gptq(H, W, s, z, 3, 8)
    np.testing.assert_array_equal(codes, grid.rtn_f32(W, s, z, 3, 8))


def test_gptq_on_grid_input_is_fixed_point():
    # Babai page 2.2: propagation after the lattice point is found changes nothing;
    # on-grid weights give zero error and their own codes.
    rng = np.random.default_rng(9)
    d_o, d_i, bits, group = 8, 32, 3, 8
    _, H = spd(d_i, rng)
    codes = rng.integers(0, 8, size=(d_o, d_i))
    codes[:, ::group] = 0
    codes[:, 1::group] = 7
    s = rng.uniform(0.005, 0.02, (d_o, d_i // group)).astype(np.float32)
    z = rng.integers(0, 8, (d_o, d_i // group)).astype(np.uint8)
    W = grid.dequant(codes, s, z, group).astype(np.float32)
    s2, z2 = grid.fit_grid_f32(W, bits, group)
    np.testing.assert_array_equal(grid.rtn_f32(W, s2, z2, bits, group), codes)
    got, _ = gptq.gptq(H, W, s2, z2, bits, group)
    np.testing.assert_array_equal(got, codes)
    assert objective.objective(H, W, grid.dequant(got, s2, z2, group)) < 1e-12


# ------------------------------------------------------------------ lattice (Babai page)
def test_babai_equals_back_to_front_gptq_200_cases():
    rng = np.random.default_rng(11)
    mism = 0
    for case in range(200):
        d = int(rng.integers(2, 12))
        X = rng.standard_normal((3 * d, d)) * rng.uniform(0.2, 3.0, d)
        H = X.T @ X + 1e-3 * np.eye(d)
        w = rng.standard_normal(d) * 0.05
        s = rng.uniform(0.01, 0.03, d)
        z = rng.integers(0, 4, d).astype(np.float64)
        order = np.arange(d)[::-1]
        cg, _ = gptq.gptq(H, w[None, :], s[:, None].T, z[None, :], 2, 1,
                          order=order, clip=False)
        cb = lattice.babai_row_cholesky(H, w, s, z) + 0
        # Babai's integers are offsets relative to code units (v includes z already)
        mism += int(np.sum(cg[0] != cb))
    assert mism == 0


def test_theorem1_any_factorisation():
    rng = np.random.default_rng(12)
    for _ in range(50):
        d = int(rng.integers(2, 10))
        X = rng.standard_normal((4 * d, d))
        w = rng.standard_normal(d) * 0.05
        s = rng.uniform(0.01, 0.03, d)
        z = rng.integers(0, 4, d).astype(np.float64)
        H = X.T @ X
        np.testing.assert_array_equal(lattice.babai_row_cholesky(H, w, s, z),
                                      lattice.babai_row_qr(X, w, s, z))


def test_ldl_diagonal_against_scipy_and_inverse_factor():
    rng = np.random.default_rng(13)
    _, H = spd(20, rng)
    D = lattice.ldl_diagonal(H)
    lu, d, perm = scipy.linalg.ldl(H, lower=True)
    np.testing.assert_allclose(np.sort(D), np.sort(np.diag(d)), rtol=1e-10)
    if np.array_equal(perm, np.arange(20)):
        np.testing.assert_allclose(D, np.diag(d), rtol=1e-10)
    # 1 / R_jj^2 equals the pivot of the reversed elimination
    R = gptq.inverse_factor(H)
    Drev = lattice.ldl_diagonal(H[::-1, ::-1])[::-1]
    np.testing.assert_allclose(1.0 / np.diag(R) ** 2, Drev, rtol=1e-9)


def test_theorem5_bound_no_clip():
    rng = np.random.default_rng(14)
    worst = 0.0
    for _ in range(100):
        d = int(rng.integers(2, 24))
        X = rng.standard_normal((3 * d, d)) * rng.uniform(0.2, 5.0, d)
        H = X.T @ X + 1e-2 * np.eye(d)
        w = rng.standard_normal(d) * 0.05
        s = rng.uniform(0.005, 0.03, d).astype(np.float32)
        z = rng.integers(0, 4, d).astype(np.uint8)
        order = rng.permutation(d) if rng.random() < 0.5 else np.arange(d)
        codes, _, E = gptq.gptq(H, w[None, :], s[None, :], z[None, :], 2, 1, order=order,
                                clip=False, return_E=True)
        e = w - grid.dequant(codes, s[None, :], z[None, :], 1)[0]
        err = e @ H @ e
        bound = lattice.theorem5_bound(H, s, order)
        assert err <= bound * (1 + 1e-9)
        worst = max(worst, err / bound)
        # elementwise: |E_j| <= s_j / (2 R_jj)
        R = gptq.inverse_factor(H[np.ix_(order, order)])
        assert np.all(np.abs(E[0]) <= s[order] / (2 * np.diag(R)) * (1 + 1e-9))
    assert worst > 0.2        # the bound is not vacuous on these cases


# ------------------------------------------------------------------ exhaustive search
def _tiny(rng, d, bits):
    X = rng.standard_normal((3 * d, d)) * rng.uniform(0.3, 3, d)
    X[:, 1] = X[:, 0] + 0.05 * rng.standard_normal(3 * d)
    H, _ = hessian.hessian(X, 0.01)
    W = (rng.standard_normal((2, d)) * 0.02).astype(np.float32)
    s, z = grid.fit_grid_f32(W, bits, d)
    return H, W, s, z


@pytest.mark.parametrize("bits,d", [(2, 8), (3, 5), (4, 4)])
def test_enumeration_bounds_solvers_from_below(bits, d):
    rng = np.random.default_rng(20 + d)
    for _ in range(3):
        H, W, s, z = _tiny(rng, d, bits)
        cg, _ = gptq.gptq(H, W, s, z, bits, d)
        rtn = grid.rtn_f32(W, s, z, bits, d)
        out = admm.admm(H, W, bits, d, 30, 0.1, 1.3, refresh_every=0)
        for r in range(2):
            sf = np.repeat(s[r], d).astype(np.float64); zf = np.repeat(z[r], d).astype(np.float64)
            best_c, best_v = lattice.enumerate_row(H, W[r], sf, zf, bits)
            for codes in (cg, rtn, out["codes"]):
                e = W[r] - sf * (codes[r] - zf)
                assert best_v <= e @ H @ e + 1e-15
            # the optimum is one of the enumerated vectors and is on the grid
            assert np.all((best_c >= 0) & (best_c < (1 << bits)))


def test_enumeration_diagonal_hessian_equals_rtn():
    rng = np.random.default_rng(30)
    d, bits = 6, 3
    H = np.diag(rng.uniform(0.5, 2, d))
    W = (rng.standard_normal((1, d)) * 0.02).astype(np.float32)
    s, z = grid.fit_grid_f32(W, bits, d)
    sf = np.repeat(s[0], d).astype(np.float64); zf = np.repeat(z[0], d).astype(np.float64)
    best_c, _ = lattice.enumerate_row(H, W[0], sf, zf, bits)
    np.testing.assert_array_equal(best_c, grid.rtn_f32(W, s, z, bits, d)[0])


# ------------------------------------------------------------------ ADMM-Q
def test_admm_w_update_eig_equals_solve():
    rng = np.random.default_rng(40)
    _, H = spd(24, rng)
    sig, Ht, lam, V = admm.spectral(H)
    Wt_hat = rng.standard_normal((5, 24))
    M = rng.standard_normal((5, 24))
    P = (Wt_hat @ V) * lam
    for rho in (1e-3, 0.05, 3.0):
        np.testing.assert_allclose(admm.w_update_eig(P, M, V, lam, rho),
                                   admm.w_update_solve(Ht, Wt_hat, M, rho), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("refresh_every", [1, 3])
def test_admm_solve_route_follows_the_eig_route(refresh_every):
    # the Cholesky-solve W-update gives the same trajectory as the eigendecomposition
    # form, also when started from a mid-run state (single-step replay)
    X, W, _ = qz_synth.tiny_layer(3)
    H, _ = hessian.hessian(X, 0.01)
    W = W[:16]
    a = admm.admm(H, W, 4, 128, 12, 0.1, 1.3, refresh_every, trace=True)
    b = admm.admm(H, W, 4, 128, 12, 0.1, 1.3, refresh_every, wupdate="solve")
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["zero"], b["zero"])
    np.testing.assert_allclose(a["scale"], b["scale"], rtol=1e-6)
    np.testing.assert_allclose(a["U"], b["U"], rtol=1e-7, atol=1e-9)
    mid = admm.admm(H, W, 4, 128, 7, 0.1, 1.3, refresh_every)
    st = dict(t0=7, codes=mid["codes"], scale=mid["scale"], zero=mid["zero"], U=mid["U"])
    c = admm.admm(H, W, 4, 128, 5, 0.1, 1.3, refresh_every, state=st, wupdate="solve")
    np.testing.assert_array_equal(c["codes"], a["codes"])
    np.testing.assert_allclose(c["U"], a["U"], rtol=1e-7, atol=1e-9)
    with pytest.raises(ValueError):
        admm.admm(H, W, 4, 128, 1, 0.1, 1.3, wupdate="lu")


def test_admm_w_update_is_penalised_minimiser():
    # gradient of (1/2)(W~-W~hat)H~(..)^T + (rho/2)||W~ - M||^2 vanishes
    rng = np.random.default_rng(41)
    _, H = spd(16, rng)
    sig, Ht, lam, V = admm.spectral(H)
    Wt_hat = rng.standard_normal((3, 16)); M = rng.standard_normal((3, 16))
    Wt = admm.w_update_eig((Wt_hat @ V) * lam, M, V, lam, 0.3)
    g = (Wt - Wt_hat) @ Ht + 0.3 * (Wt - M)
    assert np.abs(g).max() < 1e-10


def test_admm_scaling_invariance():
    # the objective in scaled coordinates equals the original one
    rng = np.random.default_rng(42)
    _, H = spd(12, rng, cond_scale=10)
    sig, Ht, _, _ = admm.spectral(H)
    A = rng.standard_normal((4, 12)) * 0.01
    B = rng.standard_normal((4, 12)) * 0.01
    f1 = objective.objective(H, A, B)
    f2 = objective.objective(Ht, A / sig, B / sig)
    assert f1 == pytest.approx(f2, rel=1e-12)


def _admm_layer(seed, d_i=32, d_o=12, bits=3, group=16):
    rng = np.random.default_rng(seed)
    _, H = spd(d_i, rng, cond_scale=6)
    W = (rng.standard_normal((d_o, d_i)) * 0.02).astype(np.float32)
    return H, W, bits, group


def test_admm_zero_iterations_is_rtn():
    H, W, bits, group = _admm_layer(43)
    out = admm.admm(H, W, bits, group, 0, 0.1, 1.3)
    s, z = grid.fit_grid_f32(W, bits, group)
    np.testing.assert_array_equal(out["codes"], grid.rtn_f32(W, s, z, bits, group))


def test_admm_huge_rho_is_rtn():
    # rho -> infinity pins W~ to D~ - U = D~^0, so the projection returns RTN(W_hat)
    H, W, bits, group = _admm_layer(44)
    s, z = grid.fit_grid_f32(W, bits, group)
    out = admm.admm(H, W, bits, group, 10, 1e12, 1.1, refresh_every=0)
    np.testing.assert_array_equal(out["codes"], grid.rtn_f32(W, s, z, bits, group))
    np.testing.assert_array_equal(out["scale"], s)
    # with the clamped refresh the grid can only narrow inside the initial range
    lo0, hi0 = grid.fit_range_f32(W, group)
    out = admm.admm(H, W, bits, group, 10, 1e12, 1.1, refresh_every=1)
    zf = out["zero"].astype(np.float64)
    sf = out["scale"].astype(np.float64)
    lo = -zf * sf
    hi = (grid.maxq(bits) - zf) * sf
    width0 = (hi0 - lo0).astype(np.float64)
    assert np.all(hi - lo <= width0 * (1 + 1e-6))


@pytest.mark.parametrize("refresh", [0, 1])
def test_admm_on_grid_input_is_fixed_point(refresh):
    rng = np.random.default_rng(45)
    d_o, d_i, bits, group = 6, 32, 3, 8
    _, H = spd(d_i, rng)
    codes = rng.integers(0, 8, size=(d_o, d_i))
    codes[:, ::group] = 0
    codes[:, 1::group] = 7
    s = rng.uniform(0.005, 0.02, (d_o, d_i // group)).astype(np.float32)
    z = rng.integers(0, 8, (d_o, d_i // group)).astype(np.uint8)
    W = grid.dequant(codes, s, z, group).astype(np.float32)
    out = admm.admm(H, W, bits, group, 25, 0.05, 1.2, refresh_every=refresh)
    np.testing.assert_array_equal(out["codes"], codes)
    sig = 1.0 / np.sqrt(np.diag(H))
    assert out["res"][-1, 0] < 1e-6 * np.linalg.norm(W / sig)


@pytest.mark.parametrize("dual", ["lagrange", "scaled"])
def test_admm_primal_residual_vanishes_under_schedule(dual):
    # ADMM-Q page, convergence: under rho_t = rho_0 gamma^t the continuous and the
    # discrete iterates reach the same limit.
    H, W, bits, group = _admm_layer(46, d_i=48, d_o=16)
    out = admm.admm(H, W, bits, group, 120, 0.05, 1.1, refresh_every=1, dual=dual)
    r = out["res"][:, 0]
    assert r[-1] <= 1e-3 * max(r[:5].max(), 1e-30) or r[-1] < 1e-8


def test_admm_warm_start_equals_single_run():
    H, W, bits, group = _admm_layer(47)
    full = admm.admm(H, W, bits, group, 12, 0.1, 1.2, refresh_every=2)
    a = admm.admm(H, W, bits, group, 5, 0.1, 1.2, refresh_every=2)
    b = admm.admm(H, W, bits, group, 7, 0.1, 1.2, refresh_every=2,
                  state=dict(t0=5, codes=a["codes"], scale=a["scale"], zero=a["zero"], U=a["U"]))
    np.testing.assert_array_equal(b["codes"], full["codes"])
    np.testing.assert_allclose(b["res"], full["res"][5:], rtol=1e-12, atol=1e-300)


def test_admm_rows_are_independent():
    H, W, bits, group = _admm_layer(48)
    full = admm.admm(H, W, bits, group, 15, 0.1, 1.2)
    part = admm.admm(H, W[3:7], bits, group, 15, 0.1, 1.2)
    np.testing.assert_array_equal(part["codes"], full["codes"][3:7])
