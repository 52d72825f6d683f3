"""GPU: ADMM-Q on the hand-derived trajectory and on a group whose refreshed range
the clamp closes (ADMM-Q page, technical summary, Methodology 2).

tests/golden/admm_trajectory.json gives three iterations on one row of four weights in
exact rational arithmetic (its notes derive every step).  The library runs them through
the C ABI (qz_admmq_prepare, then qz_admmq one iteration at a time with
QZ_ADMM_WARM_START, and once uninterrupted): codes and zero points must equal the
derivation's, refreshed scales within 1e-5 relative (the library forms the range in
fp32), the dual U within 1e-5 of max |W_hat / sigma| and the residuals within 1e-4
relative (fp32 matrix-core products)."""
from fractions import Fraction

import numpy as np
import pytest

from conftest import golden
from gpu_util import qz, report, to_dev, to_host

pytestmark = pytest.mark.gpu

G = golden("admm_trajectory.json")


def fr(x):
    return float(Fraction(x))


@pytest.mark.parametrize("name", ["A", "B"])
def test_gpu_admm_follows_hand_derived_trajectory(name):
    q = qz()
    c = next(c for c in G["cases"] if c["name"] == name)
    bits, group, refresh = G["bits"], G["group"], G["refresh_every"]
    rho0, gamma = fr(c["rho0"]), fr(c["gamma"])
    H = np.array(G["H"], np.float32)
    W = np.array([[fr(x) for x in c["W_hat"]]], np.float32)
    sig_ref = np.array([fr(x) for x in G["sigma"]], np.float32)
    V, lam, sig = q.qz_admmq_prepare(to_dev(H))
    np.testing.assert_array_equal(to_host(sig), sig_ref)
    Wd = to_dev(W)
    wmax = float(np.abs(W[0] / sig_ref).max())
    print(f"[admm_golden] case {name}: rho0={rho0} gamma={gamma}", flush=True)
    st = q.qz_admmq(V, lam, sig, Wd, bits, group, 0, rho0, gamma, refresh)
    ini = c["initial"]
    assert to_host(st["codes"])[0].tolist() == ini["codes"]
    assert int(to_host(st["zeros"])[0, 0]) == ini["zero"]
    assert float(to_host(st["scales"])[0, 0]) == fr(ini["scale"])
    res = []
    for g in c["steps"]:
        o = q.qz_admmq(V, lam, sig, Wd, bits, group, 1, rho0, gamma, refresh, t0=g["t"], state=st)
        t = g["t"]
        assert to_host(st["codes"])[0].tolist() == g["codes"], f"codes at t={t}"
        assert int(to_host(st["zeros"])[0, 0]) == g["zero"], f"zero at t={t}"
        np.testing.assert_allclose(to_host(st["scales"])[0, 0], fr(g["scale"]), rtol=1e-5,
                                   err_msg=f"scale at t={t}")
        np.testing.assert_allclose(to_host(st["U"])[0], [fr(x) for x in g["U"]], rtol=0,
                                   atol=1e-5 * wmax, err_msg=f"U at t={t}")
        res.append(to_host(o["residuals"])[0])
    want = np.sqrt([[fr(g["r_p_sq"]), fr(g["r_d_sq"])] for g in c["steps"]])
    np.testing.assert_allclose(np.array(res), want, rtol=1e-4)
    full = q.qz_admmq(V, lam, sig, Wd, bits, group, G["iters"], rho0, gamma, refresh)
    for k in ("codes", "scales", "zeros", "U"):
        np.testing.assert_array_equal(to_host(full[k]), to_host(st[k]))
    report(f"admm_golden_{name}", codes=to_host(full["codes"])[0].tolist(),
           scale=float(to_host(full["scales"])[0, 0]))


def test_gpu_admm_refresh_keeps_grid_when_clamp_closes_range():
    """Non-negative weights (lo_0 = 0) and a warm-start dual that drives the whole
    continuous iterate below 0: the clamped range is [0, 0], so the group keeps its grid
    and the codes round on it; with H = I the iterate is (W_hat + rho (D - U)) / (1 + rho)."""
    q = qz()
    import torch
    W = np.array([[0.0625, 0.1875, 0.3125, 0.5]], np.float32)
    H = np.eye(4, dtype=np.float32)
    bits, group, rho = 2, 4, 8.0
    V, lam, sig = q.qz_admmq_prepare(to_dev(H))
    Wd = to_dev(W)
    st = q.qz_admmq(V, lam, sig, Wd, bits, group, 0, rho, 1.0, 1)
    s0 = to_host(st["scales"]).copy()
    z0 = to_host(st["zeros"]).copy()
    c0 = to_host(st["codes"]).astype(np.float64)
    assert int(z0[0, 0]) == 0
    st["U"] = torch.ones_like(st["U"])
    q.qz_admmq(V, lam, sig, Wd, bits, group, 1, rho, 1.0, 1, t0=0, state=st)
    np.testing.assert_array_equal(to_host(st["scales"]), s0)
    np.testing.assert_array_equal(to_host(st["zeros"]), z0)
    D = np.float64(s0[0, 0]) * (c0 - float(z0[0, 0]))
    Wt = (W.astype(np.float64) + rho * (D - 1.0)) / (1.0 + rho)
    assert (Wt < 0).all()
    u = (Wt + 1.0) / np.float64(s0[0, 0])
    assert np.abs(u - np.floor(u) - 0.5).min() > 0.1          # no rounding boundary nearby
    want = np.clip(np.rint(u) + float(z0[0, 0]), 0, 3)
    assert to_host(st["codes"])[0].tolist() == want[0].astype(int).tolist()
    assert np.isfinite(to_host(st["U"])).all()
