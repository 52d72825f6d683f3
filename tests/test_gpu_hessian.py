"""GPU parity: H = X^T X + lambda I against the fp64 oracle.

Tolerance (fp32 accumulation of n bf16 products, exact products):
|H_gpu - H_ref|_ij <= 4 u32 sqrt(n) sqrt(G_ii G_jj), u32 = 2^-24."""
import numpy as np
import pytest

import qz_synth
from gpu_util import qz, report, to_dev, to_host
from layer_parity import U32
from layer_parity import check_hessian as _check
from oracle import hessian

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,d", [(3000, 200), (512, 128), (4096, 77), (64, 8), (130, 300)])
def test_hessian_bf16_small(n, d):
    q = qz()
    X = qz_synth.calib_bf16(5, n, d, p_out=0.02, f_out=30.0)
    out = q.qz_build_hessian(to_dev(X), damp=0.01)
    G = hessian.gram(X)
    w = _check(to_host(out["H"]), G, n, float(to_host(out["lam"])[0]), 0.01,
               to_host(out["diag"]), to_host(out["sigma"]))
    report("hessian_bf16", n=n, d=d, worst_over_tol=f"{w:.3g}")


def test_hessian_fp32_tiny():
    q = qz()
    X, _, _ = qz_synth.tiny_layer(1)
    out = q.qz_build_hessian(to_dev(X), damp=0.01)
    G = hessian.gram(X)
    _check(to_host(out["H"]), G, X.shape[0], float(to_host(out["lam"])[0]), 0.01)


def test_hessian_chunked_accumulation():
    q = qz()
    import torch
    X = qz_synth.calib_bf16(6, 5000, 136)
    Xd = to_dev(X)
    H = torch.empty((136, 136), dtype=torch.float32, device="cuda")
    q.qz_build_hessian(Xd[:2048], flags=q.QZ_H_NO_FINALIZE, H=H)
    q.qz_build_hessian(Xd[2048:4000], flags=q.QZ_H_ACCUMULATE | q.QZ_H_NO_FINALIZE, H=H)
    out = q.qz_build_hessian(Xd[4000:], flags=q.QZ_H_ACCUMULATE, H=H)
    _check(to_host(out["H"]), hessian.gram(X), 5000, float(to_host(out["lam"])[0]), 0.01)


def test_hessian_no_finalize_leaves_raw_upper():
    q = qz()
    X = qz_synth.calib_bf16(7, 1000, 150)
    out = q.qz_build_hessian(to_dev(X), flags=q.QZ_H_NO_FINALIZE)
    H = to_host(out["H"]).astype(np.float64)
    G = hessian.gram(X)
    iu = np.triu_indices(150)
    g = np.sqrt(np.outer(np.diag(G), np.diag(G)))
    assert np.all(np.abs(H - G)[iu] <= 4 * U32 * np.sqrt(1000) * g[iu])


def test_hessian_empty_calibration():
    q = qz()
    import torch
    out = q.qz_build_hessian(torch.empty((0, 40), dtype=torch.bfloat16, device="cuda"))
    assert not to_host(out["H"]).any()


def test_hessian_deterministic():
    q = qz()
    X = to_dev(qz_synth.calib_bf16(8, 3000, 264))
    a = to_host(q.qz_build_hessian(X)["H"])
    b = to_host(q.qz_build_hessian(X)["H"])
    np.testing.assert_array_equal(a, b)


def test_hessian_full_size_sampled():
    """Headline shape: 262144 tokens x 4096 channels; a 64-channel sub-block (outlier
    channels included) and the damping against fp64 sums over all tokens."""
    q = qz()
    import torch
    n, d = 262144, 4096
    X = qz_synth.calib_bf16_torch(4, n, d, p_out=0.01, f_out=30.0)
    out = q.qz_build_hessian(X, damp=0.01)
    H = out["H"]
    ch = qz_synth.outlier_channels(4, d, 0.01)
    S = np.unique(np.concatenate([ch[:16], np.random.default_rng(0).choice(d, 48, replace=False)]))
    St = torch.from_numpy(S).cuda()
    Xs = to_host(X[:, St].contiguous())
    Gs = hessian.gram(Xs, chunk=1 << 16)
    # diag of X^T X over every channel for lambda: column sums of squares in fp64
    dsum = np.zeros(d)
    for a in range(0, n, 16384):
        xb = to_host(X[a:a + 16384])
        xf = hessian.bf16_to_f64(xb)
        dsum += (xf * xf).sum(0)
    lam = 0.01 * dsum.mean()
    lam_gpu = float(to_host(out["lam"])[0])
    assert abs(lam_gpu - lam) <= 1e-5 * lam
    Hs = to_host(H[St][:, St]).astype(np.float64)
    ref = Gs + lam * np.eye(len(S))
    g = np.sqrt(np.outer(np.diag(Gs), np.diag(Gs)))
    worst = float((np.abs(Hs - ref) / (4 * U32 * np.sqrt(n) * g)).max())
    report("hessian_full", n=n, d=d, sampled=len(S), worst_over_tol=f"{worst:.3g}")
    assert worst <= 1.0
    Hh = to_host(H)
    np.testing.assert_array_equal(Hh, Hh.T)
