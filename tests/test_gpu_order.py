"""GPU parity of the quantization orders (qz_order), the no-clip error bound
(qz_error_bound) and GPTQ without clipping (qz_gptq_noclip, qz_objective with int32
codes) against the oracle.  H and the grids come from the oracle.

The min-pivot order is an integer result decided in fp64 on both sides: the oracle
follows the GPU's choice only where the GPU's pivot is within 1e-9 of the largest
diagonal entry of the smallest candidate (the rounding resolution of Schur complements
after many eliminations); such adoptions are counted.  At the full layer size the
oracle's plain elimination is too slow, so the GPU's order is checked there through a
LAPACK Cholesky of H reordered by it: its pivots must equal the GPU's, and at every
step the chosen pivot must be the smallest Schur diagonal (within the same 1e-9)."""
import numpy as np
import pytest

import qz_synth
from gpu_util import TOL_OBJECTIVE, qz, report, to_dev, to_host
from layer_parity import sample_rows
from oracle import gptq, grid, hessian, objective, order

pytestmark = pytest.mark.gpu

TIE = 1e-9      # relative to the largest diagonal entry


def _spd(seed, d, n=None, dup=False):
    X = qz_synth.calib_bf16(seed, 4 * d if n is None else n, d, p_out=0.03, f_out=20.0)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    if dup:     # exactly equal diagonal entries: the tie rules
        Hf[5, 5] = Hf[9, 9]
        Hf[17, 17] = Hf[9, 9]
    return Hf


@pytest.mark.parametrize("seed,d,dup", [(1, 96, True), (2, 200, False), (3, 333, True), (4, 1, False)])
def test_act_order_matches_oracle(seed, d, dup):
    q = qz()
    Hf = _spd(seed, d, dup=dup and d > 20)
    perm = to_host(q.qz_order(to_dev(Hf), "act")).astype(np.int64)
    np.testing.assert_array_equal(perm, order.act_order(Hf.astype(np.float64)))


@pytest.mark.parametrize("seed,d,dup", [(5, 96, True), (6, 200, False), (7, 333, False), (8, 64, False),
                                        (9, 65, True), (10, 1, False)])
def test_min_pivot_order_matches_oracle(seed, d, dup):
    q = qz()
    Hf = _spd(seed, d, dup=dup)
    perm, piv = q.qz_order(to_dev(Hf), "min_pivot", pivots=True)
    perm, piv = to_host(perm).astype(np.int64), to_host(piv)
    H64 = Hf.astype(np.float64)
    tol = TIE * float(np.max(np.diag(H64)))
    ref, D, adopted = order.min_pivot_order(H64, hint=perm, tol=tol)
    report("min_pivot", d=d, adopted=adopted)
    np.testing.assert_array_equal(perm, ref)
    np.testing.assert_allclose(piv, D, rtol=1e-9, atol=tol)
    assert adopted <= max(1, d // 100)


def test_min_pivot_diagonal_hessian_is_act_order():
    q = qz()
    rng = np.random.default_rng(11)
    dg = rng.uniform(0.5, 3.0, 150).astype(np.float32)
    dg[[3, 40, 77]] = dg[10]
    Hf = np.diag(dg).astype(np.float32)
    perm = to_host(q.qz_order(to_dev(Hf), "min_pivot")).astype(np.int64)
    act = to_host(q.qz_order(to_dev(Hf), "act")).astype(np.int64)
    np.testing.assert_array_equal(perm, act)
    np.testing.assert_array_equal(act, order.act_order(Hf.astype(np.float64)))


def _check_greedy_by_cholesky(H64, perm, piv):
    """Pivots of the GPU's order from a LAPACK Cholesky of H reordered with the column
    quantized last first; at every elimination step the chosen pivot is the smallest
    remaining Schur diagonal."""
    n = H64.shape[0]
    elim = perm[::-1]
    L = np.linalg.cholesky(H64[np.ix_(elim, elim)])
    Dl = np.diag(L) ** 2                         # pivots in elimination order
    tol = TIE * float(np.max(np.diag(H64)))
    np.testing.assert_allclose(piv[::-1], Dl, rtol=1e-8, atol=tol)
    # Schur diagonal of position q after t eliminations: H_qq - sum_{c<t} L_qc^2
    hd = np.diag(H64)[elim]
    worst = 0.0
    csum = np.zeros(n)
    L2 = L * L
    for t in range(n - 1):
        rest = hd[t + 1:] - csum[t + 1:]        # candidates not chosen at step t
        gap = Dl[t] - rest.min()
        worst = max(worst, gap / tol)
        csum += L2[:, t]
    return worst


def test_min_pivot_order_full_layer_size():
    import torch
    q = qz()
    cfg = qz_synth.WORKLOADS["up_4096x12288_w3g128"]
    X = qz_synth.calib_bf16_torch(cfg["seed"], 16384, cfg["d_i"], cfg["p_out"], cfg["f_out"])
    Xh = to_host(X)
    del X
    torch.cuda.empty_cache()
    H64, _ = hessian.hessian(Xh, cfg["damp"])
    Hf = H64.astype(np.float32)
    H64 = Hf.astype(np.float64)
    Hd = to_dev(Hf)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    perm, piv = q.qz_order(Hd, "min_pivot", pivots=True)
    ev1.record()
    torch.cuda.synchronize()
    perm, piv = to_host(perm).astype(np.int64), to_host(piv)
    np.testing.assert_array_equal(np.sort(perm), np.arange(cfg["d_i"]))
    worst = _check_greedy_by_cholesky(H64, perm, piv)
    act = to_host(q.qz_order(Hd, "act")).astype(np.int64)
    np.testing.assert_array_equal(act, order.act_order(H64))
    report("min_pivot_full", d=cfg["d_i"], ms=ev0.elapsed_time(ev1), worst_gap_over_tol=worst,
           trace_D=float(piv.sum()), same_as_act=float(np.mean(perm == act)))
    assert worst <= 1.0


@pytest.mark.parametrize("which", ["natural", "act", "min_pivot"])
def test_error_bound_matches_oracle(which):
    q = qz()
    Hf = _spd(12, 256)
    H64 = Hf.astype(np.float64)
    W = (np.random.default_rng(13).standard_normal((40, 256)) * 0.02).astype(np.float32)
    s, z = grid.fit_grid_f32(W, 3, 32)
    Hd = to_dev(Hf)
    perm = None if which == "natural" else q.qz_order(Hd, which)
    total, rows = q.qz_error_bound(Hd, to_dev(s), 32, perm=perm, rows=True)
    p = np.arange(256) if perm is None else to_host(perm).astype(np.int64)
    ref = order.layer_bound(H64, s, 32, p)
    np.testing.assert_allclose(to_host(rows), ref, rtol=1e-8)
    assert abs(total - ref.sum()) <= 1e-8 * ref.sum()


def test_error_bound_full_layer_size():
    """The 4096-column layer: per-row bounds of sampled rows in the natural, act and
    min-pivot orders against pivots from a LAPACK Cholesky of H reordered with the
    column quantized last first (the oracle's plain elimination is too slow here)."""
    import torch
    q = qz()
    cfg = qz_synth.WORKLOADS["up_4096x12288_w3g128"]
    X = qz_synth.calib_bf16_torch(cfg["seed"], 16384, cfg["d_i"], cfg["p_out"], cfg["f_out"])
    Xh = to_host(X)
    del X
    torch.cuda.empty_cache()
    H64, _ = hessian.hessian(Xh, cfg["damp"])
    Hf = H64.astype(np.float32)
    H64 = Hf.astype(np.float64)
    W = qz_synth.weights_bf16(cfg["seed"], cfg["d_o"], cfg["d_i"])
    Wf = qz_synth.bf16_bits_to_f32(W)
    s, _ = grid.fit_grid_f32(Wf, cfg["bits"], cfg["group"])
    Hd, sd = to_dev(Hf), to_dev(s)
    rows = sample_rows(cfg["d_o"])
    n, g = cfg["d_i"], cfg["group"]
    totals = {}
    for which in ("natural", "act", "min_pivot"):
        perm_d = None if which == "natural" else q.qz_order(Hd, which)
        perm = np.arange(n) if perm_d is None else to_host(perm_d).astype(np.int64)
        total, b = q.qz_error_bound(Hd, sd, g, perm=perm_d, rows=True)
        elim = perm[::-1]
        D = (np.diag(np.linalg.cholesky(H64[np.ix_(elim, elim)])) ** 2)[::-1]
        sc = s[:, perm // g].astype(np.float64)
        ref = 0.125 * (sc * sc) @ D
        np.testing.assert_allclose(to_host(b)[rows], ref[rows], rtol=1e-8)
        assert abs(total - ref.sum()) <= 1e-8 * ref.sum()
        totals[which] = total
    report("error_bound_full", **totals)


@pytest.mark.parametrize("which,bits,group,d_o,d_i", [("natural", 2, 32, 64, 128),
                                                      ("act", 2, 8, 70, 200),
                                                      ("min_pivot", 3, 64, 33, 192),
                                                      ("min_pivot", 2, 128, 64, 128)])
def test_gptq_noclip_matches_oracle(which, bits, group, d_o, d_i):
    """Codes equal the oracle's no-clip GPTQ (boundary rule), some leave the grid's
    range, every row is within its Theorem 5 bound, and the int32 objective matches."""
    import torch
    q = qz()
    rng = np.random.default_rng(14 + d_i)
    Hf = _spd(15 + d_i, d_i)
    H64 = Hf.astype(np.float64)
    W = (rng.standard_normal((d_o, d_i)) * 0.02).astype(np.float32)
    W[:, ::17] *= 4.0          # heavier columns: the compensation pushes codes off the grid
    Hd, Wd = to_dev(Hf), to_dev(W)
    perm_d = None if which == "natural" else q.qz_order(Hd, which)
    perm = np.arange(d_i) if perm_d is None else to_host(perm_d).astype(np.int64)
    codes, s, zz = q.qz_gptq_noclip(Hd, Wd, bits, group, B=32, perm=perm_d)
    assert codes.dtype == torch.int32
    c = to_host(codes).astype(np.int64)
    s_h, z_h = to_host(s), to_host(zz)
    s_ref, z_ref = grid.fit_grid_f32(W, bits, group)
    np.testing.assert_array_equal(s_h, s_ref)
    np.testing.assert_array_equal(z_h, z_ref)
    ref, adopted = gptq.gptq(H64, W, s_ref, z_ref, bits, group, order=perm, clip=False, hint=c)
    np.testing.assert_array_equal(c, ref)
    assert adopted <= max(2, 1e-3 * c.size)
    off = float(np.mean((c < 0) | (c > (1 << bits) - 1)))
    f_ref = objective.row_objective(H64, W, grid.dequant(ref, s_ref, z_ref, group))
    f_gpu, rows = q.qz_objective(Hd, Wd, codes, s, zz, group, rows=True)
    np.testing.assert_allclose(to_host(rows), f_ref, rtol=TOL_OBJECTIVE, atol=TOL_OBJECTIVE * f_ref.mean())
    bound_total, bound_rows = q.qz_error_bound(Hd, s, group, perm=perm_d, rows=True)
    b = to_host(bound_rows)
    report("gptq_noclip", order=which, bits=bits, adopted=adopted, off_grid=off,
           f_over_bound=float(f_ref.sum() / bound_total))
    assert off > 0
    assert np.all(f_ref <= b * (1 + 1e-9))


def test_noclip_full_layer_rows_within_bound():
    """The headline layer shape in the min-pivot order: every row of the GPU's no-clip
    result within the GPU's per-row bound (a property at any size), sampled rows' codes
    against the oracle with the LAPACK factor of the reordered H."""
    import torch
    q = qz()
    cfg = qz_synth.WORKLOADS["up_4096x12288_w3g128"]
    X = qz_synth.calib_bf16_torch(cfg["seed"], 16384, cfg["d_i"], cfg["p_out"], cfg["f_out"])
    Xh = to_host(X)
    del X
    torch.cuda.empty_cache()
    H64, _ = hessian.hessian(Xh, cfg["damp"])
    Hf = H64.astype(np.float32)
    H64 = Hf.astype(np.float64)
    W = qz_synth.weights_bf16(cfg["seed"], cfg["d_o"], cfg["d_i"])
    Hd, Wd = to_dev(Hf), to_dev(W)
    perm_d = q.qz_order(Hd, "min_pivot")
    bits, group, B = cfg["bits"], cfg["group"], cfg["B"]
    codes, s, zz = q.qz_gptq_noclip(Hd, Wd, bits, group, B=B, perm=perm_d)
    f_tot, f_rows = q.qz_objective(Hd, Wd, codes, s, zz, group, rows=True)
    b_tot, b_rows = q.qz_error_bound(Hd, s, group, perm=perm_d, rows=True)
    fr, br = to_host(f_rows), to_host(b_rows)
    assert np.all(fr <= br * (1 + 1e-6))
    cg, sg, zg = q.qz_gptq(Hd, Wd, bits, group, B=B, perm=perm_d)
    f_clip = q.qz_objective(Hd, Wd, cg, sg, zg, group)
    rows = sample_rows(cfg["d_o"])
    perm = to_host(perm_d).astype(np.int64)
    Wf = qz_synth.bf16_bits_to_f32(W[rows])
    c = to_host(codes)[rows].astype(np.int64)
    R = gptq.inverse_factor_lapack(H64[np.ix_(perm, perm)])
    ref, adopted = gptq.gptq(None, Wf, to_host(s)[rows], to_host(zz)[rows], bits, group,
                             order=perm, clip=False, hint=c, R=R)
    off = float(np.mean((to_host(codes) < 0) | (to_host(codes) > (1 << bits) - 1)))
    report("gptq_noclip_full", f_noclip=f_tot, bound=b_tot, f_over_bound=f_tot / b_tot,
           f_clip=f_clip, off_grid=off, adopted=adopted)
    np.testing.assert_array_equal(c, ref)
    assert adopted <= 1e-3 * c.size
