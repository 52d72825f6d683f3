"""GPU parity of the pairwise-swap local search (qz_local_search) against the oracle.

Both sides start from the oracle's round-to-nearest codes on the oracle's grid and H
(no oracle input comes from the GPU).  The library forms the gradient once and then
updates it with the accepted moves, so the trajectory is observed by calls of k steps
from the same start, k = 1, 2, ... (the search is deterministic per row): the codes after
the k-step call are the state after step k.  For every step the oracle takes the same
step from the GPU's previous state, with the gradient recomputed in fp64, and must reach
the GPU's codes, adopting the GPU's choice only where its own decision margin (a
proposal within the tolerance of the best, or a running change within the tolerance of
zero) is below the fp32 resolution of the change: tol = 1e-4 s^2 max_j sum_k |H_jk| per
row.  The whole run is also replayed by the oracle alone (with the same adoption rule)
and must end on the same codes and objective."""
import numpy as np
import pytest

import qz_synth
from gpu_util import TOL_OBJECTIVE, qz, report, to_dev, to_host
from layer_parity import sample_rows
from oracle import grid, hessian, local_search as ls, objective

pytestmark = pytest.mark.gpu


def _tol(H64, s):
    return 1e-4 * float(np.max(s)) ** 2 * float(np.max(np.sum(np.abs(H64), axis=1)))


def _run(Hf, W_bits_or_f32, bits, group, steps, rows=None):
    import torch
    q = qz()
    Wf = qz_synth.bf16_bits_to_f32(W_bits_or_f32) if W_bits_or_f32.dtype == np.uint16 else W_bits_or_f32
    s, z = grid.fit_grid_f32(Wf, bits, group)
    c0 = grid.rtn_f32(Wf, s, z, bits, group).astype(np.uint8)
    Hd, Wd = to_dev(Hf), to_dev(W_bits_or_f32)
    sd, zd, cd = to_dev(s), to_dev(z), to_dev(c0)
    r = np.arange(Wf.shape[0]) if rows is None else rows
    rt = torch.from_numpy(r).cuda()
    snaps = [c0[r].astype(np.int64)]
    moved = []
    for k in range(1, steps + 1):
        cd.copy_(to_dev(c0))
        n, mv = q.qz_local_search(Hd, Wd, cd, sd, zd, bits, group, k)
        assert mv[:len(moved)] == moved[:len(mv)], "a longer run must repeat the shorter one"
        moved = list(mv)
        snaps.append(to_host(cd[rt]).astype(np.int64))
        if n < k:
            break
    return Wf, s, z, snaps, moved


def _check(name, Hf, Wf, s, z, bits, group, snaps, rows):
    H64 = Hf.astype(np.float64)
    adopted, n_moves = 0, 0
    for i, r in enumerate(rows):
        tol = _tol(H64, s[r])
        for t in range(len(snaps) - 1):
            new, acc, ad = ls.step_row(H64, Wf[r], snaps[t][i], s[r], z[r], bits, group,
                                       hint=snaps[t + 1][i], tol=tol)
            adopted += ad
            n_moves += len(acc)
            np.testing.assert_array_equal(new, snaps[t + 1][i], err_msg=f"row {r} step {t}")
        out = ls.local_search(H64, Wf[r][None, :], snaps[0][i][None, :], s[r][None, :], z[r][None, :],
                              bits, group, len(snaps) - 1, hints=[sn[i][None, :] for sn in snaps[1:]],
                              tol=tol)
        np.testing.assert_array_equal(out["codes"][0], snaps[-1][i])
    f0 = objective.row_objective(H64, Wf[rows], grid.dequant(snaps[0], s[rows], z[rows], group))
    f1 = objective.row_objective(H64, Wf[rows], grid.dequant(snaps[-1], s[rows], z[rows], group))
    report("local_search", layer=name, rows=len(rows), steps=len(snaps) - 1, moves=n_moves,
           adopted=adopted, f_after_over_before=float(f1.sum() / f0.sum()))
    assert np.all(f1 <= f0 * (1 + 1e-12))
    assert adopted <= max(2, 0.05 * n_moves)
    return f0, f1


@pytest.mark.parametrize("bits,group", [(4, 128), (3, 32), (2, 64)])
def test_local_search_tiny(bits, group):
    X, W, _ = qz_synth.tiny_layer(1)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    Wf, s, z, snaps, moved = _run(Hf, W, bits, group, 40)
    rows = np.arange(W.shape[0])
    _check(f"tiny_w{bits}g{group}", Hf, Wf, s, z, bits, group, snaps, rows)
    assert moved[0] > 0
    assert moved[-1] == 0 or len(moved) == 40


def test_local_search_full_layer_sampled_rows():
    import torch
    cfg = qz_synth.WORKLOADS["up_4096x12288_w3g128"]
    X = qz_synth.calib_bf16_torch(cfg["seed"], 16384, cfg["d_i"], cfg["p_out"], cfg["f_out"])
    Xh = to_host(X)
    del X
    torch.cuda.empty_cache()
    H, _ = hessian.hessian(Xh, cfg["damp"])
    Hf = H.astype(np.float32)
    W = qz_synth.weights_bf16(cfg["seed"], cfg["d_o"], cfg["d_i"])
    rows = sample_rows(cfg["d_o"])
    Wf, s, z, snaps, moved = _run(Hf, W, cfg["bits"], cfg["group"], 6, rows=rows)
    Wf = qz_synth.bf16_bits_to_f32(W)
    _check("up_4096x12288_w3g128", Hf, Wf, s, z, cfg["bits"], cfg["group"], snaps, rows)
    assert moved[0] > 0


def test_local_search_ragged_width():
    """d_i not a multiple of 4 (the gradient update's scalar path), 3 groups of 30."""
    X, W, _ = qz_synth.tiny_layer(3)
    X, W = np.ascontiguousarray(X[:, :90]), np.ascontiguousarray(W[:, :90])
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    Wf, s, z, snaps, moved = _run(Hf, W, 3, 30, 40)
    _check("tiny_90_w3g30", Hf, Wf, s, z, 3, 30, snaps, np.arange(W.shape[0]))
    assert moved[0] > 0


def test_local_search_long_run_matches_oracle():
    """One call to convergence against the oracle's own run to convergence (no hints):
    equal objective within 1e-4 and almost all codes equal."""
    q = qz()
    X, W, _ = qz_synth.tiny_layer(4)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    s, z = grid.fit_grid_f32(W, 3, 32)
    c0 = grid.rtn_f32(W, s, z, 3, 32).astype(np.uint8)
    cd = to_dev(c0)
    n, mv = q.qz_local_search(to_dev(Hf), to_dev(W), cd, to_dev(s), to_dev(z), 3, 32, 200)
    assert 0 < n < 200 and mv[n] == 0
    H64 = Hf.astype(np.float64)
    out = ls.local_search(H64, W, c0, s, z, 3, 32, 200)
    g = to_host(cd).astype(np.int64)
    f_gpu = objective.row_objective(H64, W, grid.dequant(g, s, z, 32)).sum()
    f_orc = objective.row_objective(H64, W, grid.dequant(out["codes"], s, z, 32)).sum()
    report("local_search_long", steps=n, moves=int(sum(mv)), oracle_steps=int(out["steps"].max()),
           f_rel=float(abs(f_gpu - f_orc) / f_orc), codes_equal=float(np.mean(g == out["codes"])))
    assert abs(f_gpu - f_orc) <= TOL_OBJECTIVE * f_orc
    assert np.mean(g == out["codes"]) >= 0.99


def test_local_search_edge_cases():
    q = qz()
    X, W, _ = qz_synth.tiny_layer(2)
    H, _ = hessian.hessian(X, 0.01)
    Hf = H.astype(np.float32)
    s, z = grid.fit_grid_f32(W, 3, 64)
    c0 = grid.rtn_f32(W, s, z, 3, 64).astype(np.uint8)
    cd = to_dev(c0)
    n, mv = q.qz_local_search(to_dev(Hf), to_dev(W), cd, to_dev(s), to_dev(z), 3, 64, 0)
    assert n == 0
    np.testing.assert_array_equal(to_host(cd), c0)
    with pytest.raises(q.QzError):
        q.qz_local_search(to_dev(Hf), to_dev(W), cd, to_dev(s), to_dev(z), 3, 128 * 2, 3)
    # on-grid weights: nothing to move
    Wq = grid.dequant(c0, s, z, 64).astype(np.float32)
    n, mv = q.qz_local_search(to_dev(Hf), to_dev(Wq), cd, to_dev(s), to_dev(z), 3, 64, 5)
    assert n == 0 and mv[0] == 0
