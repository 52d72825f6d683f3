"""GPU parity: the layer objective f = 1/2 sum_r (q_r - w_r)^T H (q_r - w_r) (qz_objective)
against the fp64 oracle, total and per row, relative 1e-4.  Codes and grids come from the
oracle's grid fit and seeded random codes, never from the GPU."""
import numpy as np
import pytest

import qz_synth
from gpu_util import qz, report, to_dev, to_host
from oracle import grid, hessian, objective

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _case(seed, d_o, d_i, group, bits, bf16):
    rng = np.random.default_rng([seed, 77])
    X = qz_synth.calib_bf16(seed, 2048, d_i, p_out=0.02, f_out=20.0)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    if bf16:
        Wb = qz_synth.weights_bf16(seed, d_o, d_i)
        W = qz_synth.bf16_bits_to_f32(Wb)
        Wd = to_dev(Wb)
    else:
        W = (rng.standard_normal((d_o, d_i)) * 0.02).astype(np.float32)
        Wd = to_dev(W)
    s, z = grid.fit_grid_f32(W, bits, group)
    codes = grid.rtn_f32(W, s, z, bits, group).astype(np.uint8)
    flip = rng.random(codes.shape) < 0.1            # perturb some codes to move off RTN
    codes = np.where(flip, np.clip(codes.astype(np.int64) + rng.choice([-1, 1], codes.shape), 0,
                                   (1 << bits) - 1), codes).astype(np.uint8)
    return Hf, W, Wd, codes, s, z


@pytest.mark.parametrize("seed,d_o,d_i,group,bits,bf16", [
    (1, 64, 128, 128, 4, False),
    (2, 70, 200, 8, 3, True),        # ragged: edge tiles in both dimensions
    (3, 300, 384, 128, 2, True),
    (4, 1, 8, 8, 8, False),
])
def test_objective_matches_oracle(seed, d_o, d_i, group, bits, bf16):
    q = qz()
    Hf, W, Wd, codes, s, z = _case(seed, d_o, d_i, group, bits, bf16)
    f, rows = q.qz_objective(to_dev(Hf), Wd, to_dev(codes), to_dev(s), to_dev(z), group, rows=True)
    H64 = Hf.astype(np.float64)
    Q = grid.dequant(codes, s, z, group)
    ref_rows = objective.row_objective(H64, W, Q)
    ref = objective.objective(H64, W, Q)
    rows = to_host(rows)
    report("objective", d_o=d_o, d_i=d_i, rel=abs(f - ref) / ref)
    assert abs(f - ref) <= TOL * ref
    np.testing.assert_allclose(rows, ref_rows, rtol=TOL, atol=TOL * ref / d_o)
    # the total is the fixed-order sum of the rows
    assert abs(f - rows.sum()) <= 1e-12 * abs(f)


def test_objective_full_layer():
    """The headline layer shape, every row, with the oracle's H from 16384 tokens."""
    q = qz()
    cfg = qz_synth.WORKLOADS["up_4096x12288_w3g128"]
    import torch
    X = qz_synth.calib_bf16_torch(cfg["seed"], 16384, cfg["d_i"], cfg["p_out"], cfg["f_out"])
    Xh = to_host(X)
    del X
    torch.cuda.empty_cache()
    H, _ = hessian.hessian(Xh, cfg["damp"])
    Hf = H.astype(np.float32)
    Wb = qz_synth.weights_bf16(cfg["seed"], cfg["d_o"], cfg["d_i"])
    W = qz_synth.bf16_bits_to_f32(Wb)
    s, z = grid.fit_grid_f32(W, cfg["bits"], cfg["group"])
    codes = grid.rtn_f32(W, s, z, cfg["bits"], cfg["group"]).astype(np.uint8)
    f = q.qz_objective(to_dev(Hf), to_dev(Wb), to_dev(codes), to_dev(s), to_dev(z), cfg["group"])
    E = grid.dequant(codes, s, z, cfg["group"]) - W.astype(np.float64)
    ref = 0.5 * float(np.sum((E @ Hf.astype(np.float64)) * E))
    report("objective_full", rel=abs(f - ref) / ref)
    assert abs(f - ref) <= TOL * ref


def test_objective_ragged_shape_with_32_deep_slabs():
    """A shape whose product has exactly 768 tiles (96 x 8) with ragged M, N and K
    (12285 x 1019 x 1019), so the matrix-core product runs its 32-deep, three-workgroup
    configuration on edge tiles with element-checked loads; rows against the oracle."""
    q = qz()
    d_o, d_i = 12285, 1019
    Hf, W, Wd, codes, s, z = _case(5, d_o, d_i, d_i, 3, True)
    f, rows = q.qz_objective(to_dev(Hf), Wd, to_dev(codes), to_dev(s), to_dev(z), d_i, rows=True)
    H64 = Hf.astype(np.float64)
    ref_rows = objective.row_objective(H64, W, grid.dequant(codes, s, z, d_i))
    report("objective_ragged768", rel=abs(f - ref_rows.sum()) / ref_rows.sum())
    np.testing.assert_allclose(to_host(rows), ref_rows, rtol=TOL, atol=TOL * ref_rows.mean())
    assert abs(f - ref_rows.sum()) <= TOL * ref_rows.sum()


def test_objective_nonfinite_weight_is_reported():
    q = qz()
    Hf, W, Wd, codes, s, z = _case(5, 16, 64, 32, 4, False)
    W = W.copy()
    W[3, 7] = np.inf
    with pytest.raises(q.QzError) as e:
        q.qz_objective(to_dev(Hf), to_dev(W), to_dev(codes), to_dev(s), to_dev(z), 32)
    assert e.value.status == -3
