"""GPU parity: ADMM-Q against the oracle.

The oracle runs the same iteration in fp64 from the same fp32 inputs (H from the
oracle, V/Lambda from its own fp64 eigendecomposition).  The GPU's per-iteration
codes and zero points, taken by resuming the GPU loop one iteration at a time
(QZ_ADMM_WARM_START; bit-identical to one uninterrupted call, checked here), serve
as boundary hints: where the oracle's pre-round value lies within 1e-4 of a rounding
boundary it follows the GPU and goes on.  Codes, zero points, scales (relative
1e-5), residuals (relative 1e-3) and objectives (relative 1e-4) are compared."""
import numpy as np
import pytest

import qz_synth
from gpu_util import TOL_OBJECTIVE, qz, report, to_dev, to_host
from oracle import admm, grid, hessian, objective

pytestmark = pytest.mark.gpu


def gpu_trace(Hf, W, bits, group, iters, rho0, gamma, refresh, flags=0):
    """One uninterrupted GPU run, and the same run resumed one iteration at a time."""
    q = qz()
    import torch
    V, lam, sig = q.qz_admmq_prepare(to_dev(Hf))
    Wd = to_dev(W)
    full = q.qz_admmq(V, lam, sig, Wd, bits, group, iters, rho0, gamma, refresh, flags=flags)
    # chained single iterations
    st = q.qz_admmq(V, lam, sig, Wd, bits, group, 0, rho0, gamma, refresh, flags=flags)
    st["U"] = torch.zeros_like(full["U"])
    codes_t, zeros_t, res = [], [], []
    for t in range(iters):
        o = q.qz_admmq(V, lam, sig, Wd, bits, group, 1, rho0, gamma, refresh, flags=flags, t0=t,
                       state=st)
        codes_t.append(to_host(st["codes"]).astype(np.int64))
        zeros_t.append(to_host(st["zeros"]).astype(np.int64))
        res.append(to_host(o["residuals"])[0])
    for k in ("codes", "scales", "zeros", "U"):
        np.testing.assert_array_equal(to_host(st[k]), to_host(full[k]))
    np.testing.assert_array_equal(np.array(res), to_host(full["residuals"]))
    return {k: to_host(v) for k, v in full.items()}, codes_t, zeros_t


def compare(H, W, bits, group, iters, rho0, gamma, refresh, flags=0, rows=None, name="admm"):
    Hf = np.asarray(H, np.float32)
    Wf = qz_synth.bf16_bits_to_f32(W) if W.dtype == np.uint16 else W
    g, codes_t, zeros_t = gpu_trace(Hf, W, bits, group, iters, rho0, gamma, refresh, flags)
    mode = "clamped"
    if flags & 0x2:
        mode = "unclamped"
    if flags & 0x4:
        mode = "from_z"
    dual = "scaled" if flags & 0x8 else "lagrange"
    r = slice(None) if rows is None else rows
    o = admm.admm(Hf.astype(np.float64), Wf[r], bits, group, iters, rho0, gamma, refresh,
                  refresh=mode, dual=dual, hints=[c[r] for c in codes_t],
                  zero_hints=[z[r] for z in zeros_t])
    H64 = Hf.astype(np.float64)
    f_gpu = objective.objective(H64, Wf[r], grid.dequant(g["codes"][r], g["scales"][r], g["zeros"][r], group))
    f_ref = objective.objective(H64, Wf[r], grid.dequant(o["codes"], o["scale"], o["zero"], group))
    report(name, adopted=o["adopted"], f_gpu=f_gpu, f_ref=f_ref,
           res_last=g["residuals"][-1].tolist() if iters else None)
    np.testing.assert_array_equal(g["codes"][r], o["codes"])
    np.testing.assert_array_equal(g["zeros"][r], o["zero"])
    # a refreshed scale is (hi - lo) / (2^b - 1) of the continuous iterate: its error is
    # the iterate's (relative to the row's magnitude), so tiny groups get an absolute floor
    np.testing.assert_allclose(g["scales"][r], o["scale"], rtol=1e-5,
                               atol=1e-5 * float(np.abs(o["scale"]).max()))
    # relative to the oracle's objective, with a floor at 1e-9 of the layer's energy
    # (1/2) sum w^T H w for layers that the grid represents almost exactly
    energy = objective.objective(H64, Wf[r], np.zeros_like(Wf[r]))
    assert abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref + 1e-9 * energy
    if rows is None and iters:
        # residuals: relative 1e-3, with a floor at fp32 resolution of the scaled weights
        # (a residual that has converged to ~0 is rounding noise on both sides)
        wt_norm = float(np.linalg.norm(Wf[r] * np.sqrt(np.diag(H64))[None, :]))
        rho = rho0 * gamma ** np.arange(iters)
        np.testing.assert_allclose(g["residuals"][:, 0], o["res"][:, 0], rtol=1e-3,
                                   atol=1e-5 * wt_norm)
        assert np.all(np.abs(g["residuals"][:, 1] - o["res"][:, 1])
                      <= 1e-3 * o["res"][:, 1] + 1e-5 * wt_norm * rho)
    return g, o


def test_admm_tiny_layer():
    X, W, _ = qz_synth.tiny_layer(1)
    H, _ = hessian.hessian(X, 0.01)
    compare(H, W, 4, 128, 20, 0.1, 1.3, 1, name="admm_tiny")


@pytest.mark.parametrize("flags", [0x2, 0x4, 0x8])
def test_admm_reading_variants(flags):
    X = qz_synth.calib_bf16(21, 2048, 128, p_out=0.02, f_out=30.0)
    H, _ = hessian.hessian(X, 0.01)
    W = qz_synth.weights_bf16(21, 40, 128)
    compare(H, W, 3, 32, 15, 0.05, 1.2, 2, flags=flags, name=f"admm_flags_{flags}")


@pytest.mark.parametrize("d_o,d_i,bits,group,refresh", [(70, 200, 3, 8, 1), (33, 256, 2, 128, 0),
                                                        (17, 96, 4, 1, 3), (9, 512, 3, 256, 1),
                                                        (12, 192, 4, 64, 2), (21, 384, 3, 128, 1),
                                                        (19, 512, 3, 128, 3), (1, 256, 2, 128, 2)])
def test_admm_ragged(d_o, d_i, bits, group, refresh):
    X = qz_synth.calib_bf16(22, 4 * d_i, d_i, p_out=0.02, f_out=30.0)
    H, _ = hessian.hessian(X, 0.01)
    W = qz_synth.weights_bf16(22, d_o, d_i)
    compare(H, W, bits, group, 12, 0.05, 1.3, refresh, name="admm_ragged")


def test_admm_zero_iterations_is_rtn():
    q = qz()
    X, W, _ = qz_synth.tiny_layer(2)
    H, _ = hessian.hessian(X, 0.01)
    V, lam, sig = q.qz_admmq_prepare(to_dev(H.astype(np.float32)))
    o = q.qz_admmq(V, lam, sig, to_dev(W), 4, 128, 0, 0.1, 1.3, 1)
    rtn, s, z = q.qz_rtn(to_dev(W), 4, 128)
    np.testing.assert_array_equal(to_host(o["codes"]), to_host(rtn))


def test_admm_prepare_matches_oracle_spectrum():
    q = qz()
    X = qz_synth.calib_bf16(23, 1024, 192, p_out=0.02, f_out=30.0)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    V, lam, sig = q.qz_admmq_prepare(to_dev(Hf))
    V, lam, sig = to_host(V).astype(np.float64), to_host(lam).astype(np.float64), to_host(sig)
    s_ref, Ht, l_ref, _ = admm.spectral(Hf.astype(np.float64))
    np.testing.assert_array_equal(sig, np.float32(1) / np.sqrt(np.diag(Hf)))
    np.testing.assert_allclose(lam, l_ref, rtol=1e-5, atol=1e-6 * l_ref.max())
    # V diag(Lambda) V^T reproduces H~ and V is orthonormal (fp32 rounding of fp64 factors)
    np.testing.assert_allclose((V * lam) @ V.T, Ht, atol=1e-5 * l_ref.max())
    np.testing.assert_allclose(V.T @ V, np.eye(192), atol=1e-5)


def test_admm_errors():
    q = qz()
    X, W, _ = qz_synth.tiny_layer(1)
    H, _ = hessian.hessian(X, 0.01)
    V, lam, sig = q.qz_admmq_prepare(to_dev(H.astype(np.float32)))
    Wn = W.copy()
    Wn[0, 0] = np.nan
    with pytest.raises(q.QzError) as e:
        q.qz_admmq(V, lam, sig, to_dev(Wn), 4, 128, 3, 0.1, 1.3, 1)
    assert e.value.status == -3
    Hn = H.astype(np.float32).copy()
    Hn[5, 5] = -1.0
    with pytest.raises(q.QzError) as e:
        q.qz_admmq_prepare(to_dev(Hn))
    assert e.value.status == -3


def test_admm_prepare_caller_workspace():
    """The eigendecomposition works in the caller's workspace: the size query, a buffer
    one byte short rejected, the exact size accepted and giving the same bytes, and two
    sizes in turn (the solver handle is kept per thread and device)."""
    q = qz()
    import torch
    for d in (96, 200):
        X = qz_synth.calib_bf16(24, 4 * d, d, p_out=0.02, f_out=30.0)
        H, _ = hessian.hessian(X, 0.01)
        Hd = to_dev(H.astype(np.float32))
        need = q.qz_admmq_prepare_workspace(d)
        assert need >= 8 * d * d
        short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
        with pytest.raises(q.QzError) as e:
            q.qz_admmq_prepare(Hd, ws=short)
        assert e.value.status == -6
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        a = q.qz_admmq_prepare(Hd, ws=ws)
        b = q.qz_admmq_prepare(Hd)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(to_host(x), to_host(y))
