"""Parity checks of one layer on sampled rows, shared by the full-shape GPU tests.

Rows of a layer are independent in both solvers (they share only H), so the oracle
runs whole sampled rows exactly as it would inside the full problem, while the GPU
solves the whole layer in the benchmark's launch configuration.  H is the oracle's
(fp64, cast to fp32 for the GPU), so no oracle input comes from the GPU except the
boundary hints: at an element whose pre-round value lies within 1e-4 of a rounding
boundary the oracle adopts the GPU's code and counts it.
"""
import numpy as np

import qz_synth
from gpu_util import TOL_OBJECTIVE, qz, report, to_dev, to_host
from oracle import admm, grid, gptq, hessian, objective

# inverse_factor (general inverse) up to this size, the LAPACK SPD route above it
_GENERAL_INVERSE_MAX = 6144
U32 = 2.0 ** -24


def check_hessian(H, G, n, lam_gpu, damp, diag=None, sigma=None):
    """GPU H against the oracle's X^T X (G, fp64) plus damping.  Tolerance for fp32
    accumulation of n exact bf16 products: |dH_ij| <= 4 u32 sqrt(n) sqrt(G_ii G_jj).
    Returns the worst error as a fraction of its tolerance."""
    d = G.shape[0]
    lam = damp * np.mean(np.diag(G))
    assert abs(lam_gpu - lam) <= 1e-5 * lam + 1e-30
    ref = G + lam * np.eye(d)
    g = np.sqrt(np.outer(np.diag(G), np.diag(G)))
    err = np.abs(H.astype(np.float64) - ref)
    tol = 4 * U32 * np.sqrt(max(n, 1)) * g + 1e-30
    worst = float((err / tol).max())
    assert worst <= 1.0, worst
    np.testing.assert_array_equal(H, H.T)
    if diag is not None:
        np.testing.assert_array_equal(diag, np.diag(H))
        np.testing.assert_array_equal(sigma, np.float32(1) / np.sqrt(diag))
    return worst


def sample_rows(d_o):
    rows = np.array([0, 1, 777, 2048, 4095])
    rows = rows[rows < d_o]
    return np.unique(np.concatenate([rows, [d_o - 1]]))


def oracle_hessian(X_bits, damp):
    """fp64 H of bf16 tokens (bit patterns) and its fp32 cast for the GPU."""
    H, _ = hessian.hessian(X_bits, damp)
    return H, H.astype(np.float32)


def oracle_R(H64):
    if H64.shape[0] <= _GENERAL_INVERSE_MAX:
        return gptq.inverse_factor(H64)
    return gptq.inverse_factor_lapack(H64)


def gptq_rows(name, Hf, W_bits, rows, bits, group, B, W_dev=None):
    """GPU GPTQ on the whole layer vs the oracle on `rows`.  Returns the sampled rows'
    objectives (gpu, oracle) and the oracle's codes."""
    q = qz()
    H64 = Hf.astype(np.float64)
    Wd = to_dev(W_bits) if W_dev is None else W_dev
    codes, s, z = q.qz_gptq(to_dev(Hf), Wd, bits, group, B)
    c_g = to_host(codes)[rows]
    s_g, z_g = to_host(s)[rows], to_host(z)[rows]
    Wf = qz_synth.bf16_bits_to_f32(W_bits[rows])
    s_ref, z_ref = grid.fit_grid_f32(Wf, bits, group)
    np.testing.assert_array_equal(s_g, s_ref)
    np.testing.assert_array_equal(z_g, z_ref)
    ref, adopted = gptq.gptq(None, Wf, s_ref, z_ref, bits, group, R=oracle_R(H64), hint=c_g)
    f_gpu = objective.row_objective(H64, Wf, grid.dequant(c_g, s_g, z_g, group))
    f_ref = objective.row_objective(H64, Wf, grid.dequant(ref, s_ref, z_ref, group))
    report("gptq_rows", layer=name, rows=len(rows), adopted=adopted,
           max_rel_f=float(np.max(np.abs(f_gpu - f_ref) / f_ref)))
    np.testing.assert_array_equal(c_g, ref)
    assert np.all(np.abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref)
    assert adopted <= 1e-3 * c_g.size
    return f_gpu, f_ref


def admm_rows_trajectory(name, Hf, W_bits, rows, bits, group, iters, rho0, gamma, refresh,
                         W_dev=None, B=128, strict=True):
    """ADMM-Q on the whole layer (one uninterrupted GPU call, and the same run resumed
    one iteration at a time, which must agree bit for bit) against the fp64 oracle on
    `rows`, twice:
      * the iteration map at every t: the oracle's step from the GPU's state at t must
        give the GPU's state at t + 1 (codes and zero points exact outside the 1e-4
        boundary band, scales relative 1e-5, the dual within 1e-5 of the largest scaled
        weight);
      * the whole run: the oracle's own trajectory (with the GPU's per-iteration codes as
        boundary hints) must end on the GPU's codes and objective (relative 1e-4).  A
        free-running fp32 trajectory can leave the fp64 one once its accumulated rounding
        moves a pre-round value across a rounding boundary by more than the band; with
        strict=False that is reported (iteration of the first departure, objective
        ratio), runs that never depart must agree to 1e-3 in objective (the refreshed
        scales' drift alone) and runs that do to 10%."""
    import torch
    q = qz()
    H64 = Hf.astype(np.float64)
    V, lam, sig = q.qz_admmq_prepare(to_dev(Hf))
    Wd = to_dev(W_bits) if W_dev is None else W_dev
    rt = torch.from_numpy(rows).cuda()
    full = q.qz_admmq(V, lam, sig, Wd, bits, group, iters, rho0, gamma, refresh)

    def snap(st):
        return dict(codes=to_host(st["codes"][rt]).astype(np.int64),
                    scale=to_host(st["scales"][rt]), zero=to_host(st["zeros"][rt]).astype(np.int64),
                    U=to_host(st["U"][rt]).astype(np.float64))

    st = q.qz_admmq(V, lam, sig, Wd, bits, group, 0, rho0, gamma, refresh)
    snaps = [snap(st)]
    for t in range(iters):
        q.qz_admmq(V, lam, sig, Wd, bits, group, 1, rho0, gamma, refresh, t0=t, state=st)
        snaps.append(snap(st))
    for k in ("codes", "scales", "zeros", "U"):
        assert torch.equal(st[k], full[k]), k
    del V, st
    Wf = qz_synth.bf16_bits_to_f32(W_bits[rows])
    spec = admm.spectral(H64)
    wt_max = float(np.abs(Wf / spec[0][None, :]).max())
    # the iteration map, every step from the GPU's state
    step_adopted, worst_u = 0, 0.0
    for t in range(iters):
        state = None if t == 0 else dict(t0=t, **snaps[t])
        nxt = snaps[t + 1]
        o1 = admm.admm(H64, Wf, bits, group, 1, rho0, gamma, refresh, state=state,
                       hints=[nxt["codes"]], zero_hints=[nxt["zero"]], spec=spec)
        step_adopted += o1["adopted"]
        np.testing.assert_array_equal(nxt["codes"], o1["codes"], err_msg=f"step {t}")
        np.testing.assert_array_equal(nxt["zero"], o1["zero"], err_msg=f"step {t}")
        np.testing.assert_allclose(nxt["scale"], o1["scale"], rtol=1e-5,
                                   atol=1e-5 * float(np.abs(o1["scale"]).max()), err_msg=f"step {t}")
        du = float(np.abs(nxt["U"] - o1["U"]).max()) / wt_max
        worst_u = max(worst_u, du)
        assert du <= 1e-5, (t, du)
    # the whole run
    o = admm.admm(H64, Wf, bits, group, iters, rho0, gamma, refresh,
                  hints=[sn["codes"] for sn in snaps[1:]], zero_hints=[sn["zero"] for sn in snaps[1:]],
                  spec=spec, trace=True)
    depart = next((t for t in range(iters) if not np.array_equal(o["trace"][t][0], snaps[t + 1]["codes"])),
                  None)
    c_g, s_g, z_g = snaps[-1]["codes"], snaps[-1]["scale"], snaps[-1]["zero"]
    f_gpu = objective.row_objective(H64, Wf, grid.dequant(c_g, s_g, z_g, group))
    f_ref = objective.row_objective(H64, Wf, grid.dequant(o["codes"], o["scale"], o["zero"], group))
    s0, z0 = grid.fit_grid_f32(Wf, bits, group)
    cg, _ = gptq.gptq(None, Wf, s0, z0, bits, group, R=oracle_R(H64))
    f_gptq = objective.row_objective(H64, Wf, grid.dequant(cg, s0, z0, group))
    report("admm_rows", layer=name, rows=len(rows), step_adopted=step_adopted,
           step_max_rel_dU=f"{worst_u:.2e}", run_adopted=o["adopted"], run_departs_at=depart,
           max_rel_f=float(np.max(np.abs(f_gpu - f_ref) / f_ref)),
           f_admm_over_f_gptq=float(f_ref.sum() / f_gptq.sum()))
    assert step_adopted <= 1e-3 * c_g.size * max(iters, 1)
    if strict:
        assert depart is None, f"trajectory departs at iteration {depart}"
        np.testing.assert_array_equal(z_g, o["zero"])
        # a refreshed scale is (hi - lo) / (2^b - 1) of the continuous iterate, whose fp32
        # deviation from the fp64 trajectory builds up over the run: relative 1e-4, the
        # floating-point tolerance of the objective
        np.testing.assert_allclose(s_g, o["scale"], rtol=TOL_OBJECTIVE,
                                   atol=TOL_OBJECTIVE * float(np.abs(o["scale"]).max()))
        assert np.all(np.abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref)
        assert o["adopted"] <= 1e-3 * c_g.size * max(iters, 1)
    else:
        if depart is None:
            # same codes all along: only the refreshed scales' fp32 drift separates them
            np.testing.assert_array_equal(z_g, o["zero"])
            assert np.all(np.abs(f_gpu - f_ref) <= 1e-3 * f_ref)
        assert abs(f_gpu.sum() - f_ref.sum()) <= 0.1 * f_ref.sum()
    return f_gpu, f_ref


def admm_rows_replay(name, Hf, W_bits, rows, bits, group, iters, rho0, gamma, refresh, ts,
                     W_dev=None, f_gptq=None):
    """The ADMM-Q iteration map at full shape, for H too large for a host
    eigendecomposition: at each t in `ts` the GPU runs one iteration of the whole layer
    and the oracle runs the same iteration on `rows` with a Cholesky solve of
    (H~ + rho_t I), both from the same state.  At t = 0 that state is the initial one,
    which the oracle computes itself (and which is compared first); at t > 0 it is the
    state the GPU reached, taken as a test point.  The objective of the final state
    (after the last listed t, plus one, iterations) is reported against GPTQ's on the
    same rows when f_gptq is given (not gated)."""
    import torch
    q = qz()
    H64 = Hf.astype(np.float64)
    sig_o = 1.0 / np.sqrt(np.diag(H64))
    Ht = H64 * sig_o[:, None]
    Ht *= sig_o[None, :]
    V, lam, sig = q.qz_admmq_prepare(to_dev(Hf))
    Wd = to_dev(W_bits) if W_dev is None else W_dev
    rt = torch.from_numpy(rows).cuda()
    Wf = qz_synth.bf16_bits_to_f32(W_bits[rows])
    wt_max = float(np.abs(Wf / sig_o[None, :]).max())

    def snap(st):
        return dict(codes=to_host(st["codes"][rt]).astype(np.int64),
                    scale=to_host(st["scales"][rt]), zero=to_host(st["zeros"][rt]).astype(np.int64),
                    U=to_host(st["U"][rt]).astype(np.float64))

    st = q.qz_admmq(V, lam, sig, Wd, bits, group, 0, rho0, gamma, refresh)
    init = snap(st)
    lo0, hi0, s0, z0, c0 = admm.initial_grid(Wf, bits, group)
    np.testing.assert_array_equal(init["codes"], c0)
    np.testing.assert_array_equal(init["scale"], s0)
    np.testing.assert_array_equal(init["zero"], z0)
    assert np.all(init["U"] == 0)
    t_cur = 0
    worst_u = 0.0
    adopted = 0
    for t in sorted(ts):
        assert t < iters
        if t > t_cur:
            q.qz_admmq(V, lam, sig, Wd, bits, group, t - t_cur, rho0, gamma, refresh, t0=t_cur, state=st)
        before = snap(st)
        q.qz_admmq(V, lam, sig, Wd, bits, group, 1, rho0, gamma, refresh, t0=t, state=st)
        t_cur = t + 1
        after = snap(st)
        state = None if t == 0 else dict(t0=t, **before)
        o = admm.admm(None, Wf, bits, group, 1, rho0, gamma, refresh, state=state,
                      hints=[after["codes"]], zero_hints=[after["zero"]], spec=(sig_o, Ht, None, None),
                      wupdate="solve")
        adopted += o["adopted"]
        np.testing.assert_array_equal(after["codes"], o["codes"])
        np.testing.assert_array_equal(after["zero"], o["zero"])
        np.testing.assert_allclose(after["scale"], o["scale"], rtol=1e-5,
                                   atol=1e-5 * float(np.abs(o["scale"]).max()))
        du = float(np.abs(after["U"] - o["U"]).max())
        worst_u = max(worst_u, du / wt_max)
        assert du <= 1e-4 * wt_max, (t, du, wt_max)
    c_g, s_g, z_g = after["codes"], after["scale"], after["zero"]
    f_gpu = objective.row_objective(H64, Wf, grid.dequant(c_g, s_g, z_g, group))
    ratio = None if f_gptq is None else float(f_gpu.sum() / np.sum(f_gptq))
    report("admm_replay", layer=name, rows=len(rows), ts=list(ts), adopted=adopted,
           max_rel_dU=worst_u, t_final=t_cur, f_admm_over_f_gptq=ratio)
    assert adopted <= 1e-3 * c_g.size * len(ts)
