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


# (5003, 520) and (2077, 776): several 256-wide tiles on the direct-copy path with a ragged
# last tile column (8 channels at d = 776) and a token count that ends inside a stage
@pytest.mark.parametrize("n,d", [(3000, 200), (512, 128), (4096, 77), (64, 8), (130, 300),
                                 (5003, 520), (2077, 776)])
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


@pytest.mark.parametrize("n,d,fp32", [(3000, 200, False), (512, 77, False), (512, 128, True)])
def test_hessian_scaled_output(n, d, fp32):
    """H_scaled = Sigma H Sigma in fp32: (H_ij sigma_i) sigma_j with the sigma output."""
    q = qz()
    if fp32:
        X = np.random.default_rng(3).standard_normal((n, d)).astype(np.float32)
    else:
        X = qz_synth.calib_bf16(9, n, d, p_out=0.02, f_out=30.0)
    out = q.qz_build_hessian(to_dev(X), damp=0.01, scaled=True)
    H, sg, Hs = to_host(out["H"]), to_host(out["sigma"]), to_host(out["H_scaled"])
    np.testing.assert_array_equal(Hs, (H * sg[:, None]) * sg[None, :])
    np.testing.assert_allclose(np.diag(Hs), 1.0, rtol=3e-7)


def test_hessian_full_size_every_entry():
    """Headline shape: 262144 tokens x 4096 channels.  Every entry of H against the
    oracle's fp64 X^T X over all tokens (host BLAS), and the damping."""
    q = qz()
    n, d = 262144, 4096
    X = qz_synth.calib_bf16_torch(4, n, d, p_out=0.01, f_out=30.0)
    out = q.qz_build_hessian(X, damp=0.01)
    H = to_host(out["H"])
    print("[hessian_full] GPU done; oracle X^T X over 262144 tokens on the host", flush=True)
    G = np.zeros((d, d))
    for a in range(0, n, 16384):
        G += hessian.gram(to_host(X[a:a + 16384]), chunk=16384)
    w = _check(H, G, n, float(to_host(out["lam"])[0]), 0.01, to_host(out["diag"]),
               to_host(out["sigma"]))
    report("hessian_full", n=n, d=d, entries=d * d, worst_over_tol=f"{w:.3g}")
