"""GPU parity for the layers with many input channels, at full shape, in the
benchmark's launch configuration, on sampled rows: the MLP down projection
12288 -> 4096 (W2 g128, 150 ADMM-Q iterations) and the 32B-like down projection
25600 -> 5120 (W3 g128, 200 iterations, grid refresh every 10).

H is the oracle's, from the first calibration tokens of the layer's own input recipe
plus the damping: 16384 tokens for the 12288-channel layer (more tokens than channels,
so H is full rank before the damping, as at the benchmark's 262144 tokens), 8192 for
the 25600-channel one (a host fp64 sum over more tokens would take many minutes; the
damping keeps it positive definite).  The GPU's full-token Hessian is checked in
test_gpu_hessian.py.

GPTQ: whole sampled rows against the oracle, R from LAPACK's SPD drivers.
ADMM-Q at 12288 channels: the whole trajectory and the map at every step, against the
oracle's fp64 eigendecomposition of H (about a minute of host LAPACK).  At 25600
channels that eigendecomposition takes over ten minutes on the host, so ADMM-Q is
checked as an iteration map there: one iteration from the initial state, and from the
state the GPU reached at later t, with a Cholesky solve of (H~ + rho_t I).
"""
import numpy as np
import pytest

import qz_synth
from gpu_util import to_host
from layer_parity import (admm_rows_replay, admm_rows_trajectory, gptq_rows, oracle_hessian,
                          sample_rows)

pytestmark = pytest.mark.gpu

N_ORACLE_TOKENS = {"mlp_down_12288x4096_w2g128": 16384, "32b_down_25600x5120_w3g128": 8192}
LAYERS = ["mlp_down_12288x4096_w2g128", "32b_down_25600x5120_w3g128"]
WHOLE_RUN = {"mlp_down_12288x4096_w2g128"}
_cache = {}


def _layer(name):
    """(cfg, Hf fp32, W bits) for one layer; only the most recent layer is kept."""
    if name not in _cache:
        _cache.clear()
        import torch
        cfg = qz_synth.WORKLOADS[name]
        X = qz_synth.calib_bf16_torch(cfg["seed"], N_ORACLE_TOKENS[name], cfg["d_i"],
                                      cfg["p_out"], cfg["f_out"])
        Xh = to_host(X)
        del X
        torch.cuda.empty_cache()
        H, Hf = oracle_hessian(Xh, cfg["damp"])
        del H, Xh
        W = qz_synth.weights_bf16(cfg["seed"], cfg["d_o"], cfg["d_i"])
        _cache[name] = dict(cfg=cfg, Hf=Hf, W=W, f_gptq=None)
    return _cache[name]


def _replay_points(cfg):
    T, k = cfg["iters"], cfg["refresh"]
    last_refresh = (T - 1) // k * k
    return sorted({0, last_refresh, T - 1})


@pytest.mark.parametrize("name", LAYERS)
def test_gptq_large_di_sampled_rows(name):
    L = _layer(name)
    cfg = L["cfg"]
    rows = sample_rows(cfg["d_o"])
    _, f_ref = gptq_rows(name, L["Hf"], L["W"], rows, cfg["bits"], cfg["group"], cfg["B"])
    L["f_gptq"] = f_ref


@pytest.mark.parametrize("name", LAYERS)
def test_admm_large_di(name):
    L = _layer(name)
    cfg = L["cfg"]
    rows = sample_rows(cfg["d_o"])
    if name in WHOLE_RUN:
        print(f"[admm_large_di] {name}: host fp64 eigendecomposition of H ({cfg['d_i']} channels)",
              flush=True)
        admm_rows_trajectory(name, L["Hf"], L["W"], rows, cfg["bits"], cfg["group"], cfg["iters"],
                             cfg["rho0"], cfg["gamma"], cfg["refresh"], B=cfg["B"])
    else:
        admm_rows_replay(name, L["Hf"], L["W"], rows, cfg["bits"], cfg["group"], cfg["iters"],
                         cfg["rho0"], cfg["gamma"], cfg["refresh"], _replay_points(cfg),
                         f_gptq=L["f_gptq"])
