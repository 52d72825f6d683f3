"""GPU parity: GPTQ against the oracle (worked examples, tiny layer, ragged shapes,
orders, error paths).

Codes must match except where the oracle's pre-round value lies within 1e-4 (code
units) of a rounding boundary; there the oracle follows the GPU's code and goes on
(boundary rule), and such adoptions are counted and reported.  Objectives (fp64,
from codes and scales) agree to 1e-4 relative.  H always comes from the oracle."""
import numpy as np
import pytest

import qz_synth
from conftest import golden
from gpu_util import TOL_OBJECTIVE, qz, report, to_dev, to_host
from oracle import gptq, grid, hessian, objective

pytestmark = pytest.mark.gpu


def _run_pair(H, W, bits, group, B, order=None, caller=None):
    """GPU GPTQ and the boundary-following oracle on the same fp32 H and W."""
    q = qz()
    Hf = np.asarray(H, np.float32)
    perm = None if order is None else to_dev(np.asarray(order, np.int32))
    kw = {}
    if caller is not None:
        kw = dict(scales=to_dev(caller[0]), zeros=to_dev(caller[1]))
    codes, s, z = q.qz_gptq(to_dev(Hf), to_dev(W), bits, group, B, perm=perm, **kw)
    codes, s, z = to_host(codes), to_host(s), to_host(z)
    Wf = qz_synth.bf16_bits_to_f32(W) if W.dtype == np.uint16 else W
    if caller is None:
        s_ref, z_ref = grid.fit_grid_f32(Wf, bits, group)
        np.testing.assert_array_equal(s, s_ref)
        np.testing.assert_array_equal(z, z_ref)
    ref, adopted = gptq.gptq(Hf.astype(np.float64), Wf, s, z, bits, group, order=order,
                             hint=codes)
    H64 = Hf.astype(np.float64)
    f_gpu = objective.objective(H64, Wf, grid.dequant(codes, s, z, group))
    f_ref = objective.objective(H64, Wf, grid.dequant(ref, s, z, group))
    return codes, ref, adopted, f_gpu, f_ref


def test_gptq_worked_example_compensation():
    g = golden("gptq_worked_examples.json")["compensation"]
    c = g["construction"]
    codes, ref, adopted, f_gpu, _ = _run_pair(np.array(g["H"]), np.array(c["W_hat"], np.float32),
                                              c["bits"], c["group"], 2,
                                              caller=(np.array(c["scale"], np.float32),
                                                      np.array(c["zero"], np.uint8)))
    np.testing.assert_array_equal(codes, c["codes_gptq"])
    assert f_gpu == pytest.approx(g["printed"]["cost_compensated"], rel=1e-6)


def test_gptq_worked_example_collinear_through_hessian():
    q = qz()
    g = golden("gptq_worked_examples.json")["collinear"]
    c = g["construction"]
    x = np.random.default_rng(3).standard_normal(64).astype(np.float32)
    X = np.stack([x, x], axis=1)
    W = np.array([g["printed"]["W_hat"]], np.float32)
    sc, zc = to_dev(np.array(c["scale"], np.float32)), to_dev(np.array(c["zero"], np.uint8))
    H = q.qz_build_hessian(to_dev(X), damp=c["damp"])["H"]
    codes, _, _ = q.qz_gptq(H, to_dev(W), c["bits"], c["group"], 2, scales=sc, zeros=zc)
    np.testing.assert_array_equal(to_host(codes), c["codes_gptq"])
    # without damping the curvature is singular: the factorisation refuses it
    H0 = q.qz_build_hessian(to_dev(X), damp=0.0)["H"]
    with pytest.raises(q.QzError) as e:
        q.qz_gptq(H0, to_dev(W), c["bits"], c["group"], 2, scales=sc, zeros=zc)
    assert e.value.status == -2


def _tiny():
    X, W, _ = qz_synth.tiny_layer(1)
    H, _ = hessian.hessian(X, 0.01)
    return H, W


def test_gptq_tiny_layer():
    H, W = _tiny()
    codes, ref, adopted, f_gpu, f_ref = _run_pair(H, W, 4, 128, 32)
    report("gptq_tiny", adopted=adopted, f_gpu=f_gpu, f_ref=f_ref)
    np.testing.assert_array_equal(codes, ref)
    assert abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref
    assert adopted <= 0.001 * codes.size


@pytest.mark.parametrize("d_o,d_i,bits,group,B", [(70, 200, 3, 8, 48), (64, 128, 2, 128, 1),
                                                   (64, 128, 3, 128, 128), (33, 384, 3, 128, 128),
                                                   (130, 256, 4, 1, 37), (5, 40, 8, 40, 16),
                                                   (40, 1100, 3, 100, 40), (24, 150, 3, 50, 32)])
def test_gptq_ragged(d_o, d_i, bits, group, B):
    X = qz_synth.calib_bf16(9, 4 * d_i, d_i, p_out=0.02, f_out=30.0)
    H, _ = hessian.hessian(X, 0.01)
    W = qz_synth.weights_bf16(9, d_o, d_i)
    codes, ref, adopted, f_gpu, f_ref = _run_pair(H, W, bits, group, B)
    report("gptq_ragged", shape=(d_o, d_i, bits, group, B), adopted=adopted, f_gpu=f_gpu, f_ref=f_ref)
    np.testing.assert_array_equal(codes, ref)
    assert abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref


@pytest.mark.parametrize("kind", ["act_order", "reversed", "random"])
def test_gptq_orders(kind):
    d_o, d_i = 48, 256
    X = qz_synth.calib_bf16(10, 1024, d_i, p_out=0.02, f_out=30.0)
    H, _ = hessian.hessian(X, 0.01)
    W = qz_synth.weights_bf16(10, d_o, d_i)
    if kind == "act_order":
        order = np.argsort(-np.diag(H), kind="stable")
    elif kind == "reversed":
        order = np.arange(d_i)[::-1].copy()
    else:
        order = np.random.default_rng(0).permutation(d_i)
    codes, ref, adopted, f_gpu, f_ref = _run_pair(H, W, 3, 32, 64, order=order)
    np.testing.assert_array_equal(codes, ref)
    assert abs(f_gpu - f_ref) <= TOL_OBJECTIVE * f_ref


def test_gptq_diagonal_hessian_equals_rtn():
    q = qz()
    d = 96
    H = np.diag(np.random.default_rng(1).uniform(0.5, 2.0, d)).astype(np.float32)
    W = qz_synth.weights_bf16(12, 16, d)
    codes, _, _ = q.qz_gptq(to_dev(H), to_dev(W), 3, 32, 32)
    rtn, _, _ = q.qz_rtn(to_dev(W), 3, 32)
    np.testing.assert_array_equal(to_host(codes), to_host(rtn))


def test_gptq_deterministic_and_errors():
    q = qz()
    H, W = _tiny()
    Hd, Wd = to_dev(H.astype(np.float32)), to_dev(W)
    a = to_host(q.qz_gptq(Hd, Wd, 4, 128, 32)[0])
    b = to_host(q.qz_gptq(Hd, Wd, 4, 128, 32)[0])
    np.testing.assert_array_equal(a, b)
    Wn = W.copy()
    Wn[3, 7] = np.inf
    with pytest.raises(q.QzError) as e:
        q.qz_gptq(Hd, to_dev(Wn), 4, 128, 32)
    assert e.value.status == -3
    with pytest.raises(q.QzError) as e:
        q.qz_gptq(Hd, Wd, 4, 128, 129)
    assert e.value.status == -1


def test_gptq_rfactor_graph_replays_follow_their_inputs():
    """The R factor is replayed from a captured graph while its arguments (pointers and
    sizes) stay the same.  Replays with the same workspace must give the codes of a fresh
    capture (a new workspace), also after the Hessian's values change in place and after
    another shape has been factored in between, with host work and synchronisation
    between the calls."""
    import torch
    q = qz()
    H, W = _tiny()
    Hd, Wd = to_dev(H.astype(np.float32)), to_dev(W)
    n_ws = q.qz_gptq_workspace(W.shape[0], W.shape[1], 32)
    ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
    X2 = qz_synth.calib_bf16(9, 1024, 256, p_out=0.02, f_out=30.0)
    H2, _ = hessian.hessian(X2, 0.01)
    W2 = qz_synth.weights_bf16(9, 48, 256)
    H2d, W2d = to_dev(H2.astype(np.float32)), to_dev(W2)
    ws2 = torch.empty(q.qz_gptq_workspace(48, 256, 64), dtype=torch.uint8, device="cuda")

    def run(Hx, Wx, bits, group, B, w):
        out = to_host(q.qz_gptq(Hx, Wx, bits, group, B, ws=w)[0])
        torch.cuda.synchronize()
        return out

    first = run(Hd, Wd, 4, 128, 32, ws)
    for _ in range(3):
        _ = torch.randn(1000, device="cuda").sum().item()   # eager work in between
        np.testing.assert_array_equal(run(Hd, Wd, 4, 128, 32, ws), first)
    other = run(H2d, W2d, 3, 32, 64, ws2)
    np.testing.assert_array_equal(run(Hd, Wd, 4, 128, 32, ws), first)
    np.testing.assert_array_equal(run(H2d, W2d, 3, 32, 64, ws2), other)
    # the Hessian changes in place: the replay reads the new values
    Hd.mul_(1.0)
    Hd[:, 3] *= 4.0
    Hd[3, :] *= 4.0
    replay = run(Hd, Wd, 4, 128, 32, ws)
    fresh = run(Hd, Wd, 4, 128, 32, torch.empty(n_ws, dtype=torch.uint8, device="cuda"))
    np.testing.assert_array_equal(replay, fresh)
    H_new = to_host(Hd).astype(np.float64)
    s, z = grid.fit_grid_f32(W, 4, 128)
    ref, _ = gptq.gptq(H_new, W, s, z, 4, 128, hint=replay)
    np.testing.assert_array_equal(replay, ref)
