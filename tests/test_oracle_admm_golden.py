"""Pins of the ADMM-Q loop as a whole (CPU only).

tests/golden/admm_trajectory.json holds three iterations of ADMM-Q on one row of four
weights, derived by hand in exact rational arithmetic (its notes give every step):
H = [[4, 2, 0, 0], [2, 4, 0, 0], [0, 0, 1, 0], [0, 0, 0, 16]], so Sigma = (1/2, 1/2, 1,
1/4) and H~ = Sigma H Sigma has a 2 x 2 block whose inverse (H~ + rho I)^-1 has a closed
form.  The oracle runs the same iterations through its eigendecomposition route in
fp64 and must land on the same codes, zero points and fp32 scales, and on the same dual
and residuals to 1e-12.  A slip in how the refresh, the projection, the dual update and
the penalty schedule interlock (ADMM-Q page, technical summary, Methodology 2) changes at
least one of them: the clamp is active, the grid narrows and two codes change in case A,
the zero point moves in case B, and the rescale rho_t / rho_(t+1) enters every U."""
from fractions import Fraction

import numpy as np
import pytest

from conftest import golden
from oracle import admm, grid

G = golden("admm_trajectory.json")


def fr(x):
    return float(Fraction(x))


def case(name):
    return next(c for c in G["cases"] if c["name"] == name)


def run_steps(c):
    """The oracle one iteration at a time (warm start), returning each step's state."""
    H = np.array(G["H"], np.float64)
    W = np.array([[fr(x) for x in c["W_hat"]]], np.float32)
    bits, group = G["bits"], G["group"]
    rho0, gamma = fr(c["rho0"]), fr(c["gamma"])
    lo0, hi0, s0, z0, c0 = admm.initial_grid(W, bits, group)
    st = dict(t0=0, codes=c0.astype(np.int64), scale=s0, zero=z0.astype(np.int64),
              U=np.zeros_like(W, dtype=np.float64))
    out = []
    for t in range(G["iters"]):
        st = dict(st, t0=t)
        r = admm.admm(H, W, bits, group, 1, rho0, gamma, G["refresh_every"], state=st)
        st = dict(t0=t + 1, codes=r["codes"], scale=r["scale"], zero=r["zero"], U=r["U"])
        out.append((r, st))
    return H, W, (lo0, hi0, s0, z0, c0), out


@pytest.mark.parametrize("name", ["A", "B"])
def test_oracle_initial_grid_matches_hand_derivation(name):
    c = case(name)
    _, _, (lo0, hi0, s0, z0, c0), _ = run_steps(c)
    ini = c["initial"]
    assert lo0[0, 0] == fr(ini["lo0"]) and hi0[0, 0] == fr(ini["hi0"])
    assert s0[0, 0] == np.float32(fr(ini["scale"])) and int(z0[0, 0]) == ini["zero"]
    assert c0[0].tolist() == ini["codes"]


@pytest.mark.parametrize("name", ["A", "B"])
def test_oracle_admm_follows_hand_derived_trajectory(name):
    c = case(name)
    _, _, _, out = run_steps(c)
    for (r, st), g in zip(out, c["steps"]):
        t = g["t"]
        assert r["codes"][0].tolist() == g["codes"], f"codes at t={t}"
        assert int(r["zero"][0, 0]) == g["zero"], f"zero at t={t}"
        # the refreshed scale is an fp32 number: it must be that exact number
        assert r["scale"].dtype == np.float32
        assert r["scale"][0, 0] == np.float32(fr(g["scale"])), f"scale at t={t}"
        assert float(r["scale"][0, 0]) == fr(g["scale"]), f"scale at t={t} is not the fp32 value"
        U = np.array([fr(x) for x in g["U"]])
        np.testing.assert_allclose(r["U"][0], U, rtol=0, atol=1e-12, err_msg=f"U at t={t}")
        rp, rd = np.sqrt(fr(g["r_p_sq"])), np.sqrt(fr(g["r_d_sq"]))
        np.testing.assert_allclose(r["res"][0], [rp, rd], rtol=1e-12, err_msg=f"residuals at t={t}")


@pytest.mark.parametrize("name", ["A", "B"])
def test_oracle_admm_uninterrupted_run_matches_hand_derivation(name):
    c = case(name)
    H = np.array(G["H"], np.float64)
    W = np.array([[fr(x) for x in c["W_hat"]]], np.float32)
    r = admm.admm(H, W, G["bits"], G["group"], G["iters"], fr(c["rho0"]), fr(c["gamma"]),
                  G["refresh_every"], trace=True)
    for (C, s, z), g in zip(r["trace"], c["steps"]):
        assert C[0].tolist() == g["codes"] and int(z[0, 0]) == g["zero"]
        assert float(s[0, 0]) == fr(g["scale"])
    last = c["steps"][-1]
    np.testing.assert_allclose(r["U"][0], [fr(x) for x in last["U"]], rtol=0, atol=1e-12)
    rs = np.sqrt([[fr(g["r_p_sq"]), fr(g["r_d_sq"])] for g in c["steps"]])
    np.testing.assert_allclose(r["res"], rs, rtol=1e-12)


def test_golden_trajectory_exercises_every_reading():
    """The fixture is only a pin if the pieces it is meant to pin are active in it."""
    a, b = case("A"), case("B")
    assert any(g["clamp_active"] for g in a["steps"]) and any(g["clamp_active"] for g in b["steps"])
    assert not b["steps"][0]["clamp_active"]
    # the grid changes at a refresh, and a code changes with the grid held by the refresh
    assert a["steps"][0]["scale"] != a["initial"]["scale"]
    assert a["steps"][1]["codes"] != a["steps"][0]["codes"]
    assert b["steps"][0]["zero"] != b["initial"]["zero"]
    # the dual is rescaled: with gamma != 1 the rescale changes every nonzero U
    for c in (a, b):
        assert fr(c["gamma"]) != 1.0 and any(fr(x) != 0 for x in c["steps"][0]["U"])


def test_admm_other_readings_leave_the_hand_derived_trajectory():
    """Each alternative reading the library offers changes the pinned trajectory, so
    the pin tells them apart (refresh off, unclamped refresh, dual without rescale,
    the schedule shifted by one iteration)."""
    c = case("A")
    H = np.array(G["H"], np.float64)
    W = np.array([[fr(x) for x in c["W_hat"]]], np.float32)
    rho0, gamma = fr(c["rho0"]), fr(c["gamma"])
    last = c["steps"][-1]
    want_U = np.array([fr(x) for x in last["U"]])

    def differs(r):
        return (r["codes"][0].tolist() != last["codes"] or
                float(r["scale"][0, 0]) != fr(last["scale"]) or
                np.abs(r["U"][0] - want_U).max() > 1e-9)

    kw = dict(bits=G["bits"], group=G["group"], iters=G["iters"], gamma=gamma)
    assert differs(admm.admm(H, W, rho0=rho0, refresh_every=0, **kw))
    assert differs(admm.admm(H, W, rho0=rho0, refresh_every=1, refresh="unclamped", **kw))
    assert differs(admm.admm(H, W, rho0=rho0, refresh_every=1, dual="scaled", **kw))
    assert differs(admm.admm(H, W, rho0=rho0 * gamma, refresh_every=1, **kw))


def test_admm_refresh_keeps_grid_when_clamp_closes_range():
    """A group of non-negative weights has lo_0 = 0; if the continuous iterate of that
    group falls entirely below 0 the clamped range is [0, 0], which defines no grid: the
    group keeps its grid (scale, zero) and the codes round on it.  With H = I (Sigma = I,
    H~ = I) the W-update is W~ = (W_hat + rho (D - U)) / (1 + rho), checked here in closed
    form."""
    W = np.array([[0.0625, 0.1875, 0.3125, 0.5]], np.float32)
    H = np.eye(4)
    bits, group, rho = 2, 4, 8.0
    lo0, hi0, s0, z0, c0 = admm.initial_grid(W, bits, group)
    assert lo0[0, 0] == 0.0
    U0 = np.full((1, 4), 1.0)
    st = dict(t0=0, codes=c0.astype(np.int64), scale=s0, zero=z0.astype(np.int64), U=U0)
    r = admm.admm(H, W, bits, group, 1, rho, 1.0, 1, state=st)
    D = grid.dequant(c0, s0, z0, group)
    Wt = (W.astype(np.float64) + rho * (D - U0)) / (1.0 + rho)
    assert (Wt < 0).all()                       # the iterate left the group's range
    assert r["scale"][0, 0] == s0[0, 0] and r["zero"][0, 0] == z0[0, 0]
    assert np.isfinite(r["U"]).all()
    want = np.clip(np.rint((Wt + U0) / np.float64(s0[0, 0])) + float(z0[0, 0]), 0, 3)
    assert r["codes"][0].tolist() == want[0].astype(int).tolist()
