"""GPU parity on a whole 8B-like decoder block quantized sub-layer by sub-layer
(q/k/v 4096 -> 4096/1024/1024 on one shared Hessian, o_proj 4096 -> 4096, gate/up
4096 -> 12288 on one shared Hessian, down 12288 -> 4096), with 262144 calibration
tokens propagated through the already-quantized sub-layers of a pre-norm decoder block
(RMSNorm, causal softmax attention per 2048-token sequence, residual add, SwiGLU; see
block_driver.py): at W3 g128 propagating ADMM-Q's result and at W4 g128 propagating
GPTQ's.

For every sub-layer, on its own propagated input: the GPU Hessian of the input's first
16384 tokens against the oracle's, entry by entry (once per shared input); then GPTQ and
ADMM-Q on the oracle's H of those tokens against the oracle on sampled rows.  ADMM-Q:
the whole trajectory and the map at every step for every sub-layer of the W3 pipeline
(down_proj's 12288 channels included: the host eigendecomposition takes about a
minute); in the W4 pipeline the same for d_i = 4096 and the iteration map for down_proj.
The propagated inputs depend on the codes of the sub-layers before them (the GPU's,
from the full-token Hessians): they are test inputs to both sides.

At 4 bits the free-running fp32 trajectory can leave the fp64 one (its rounding moves a
pre-round value across a boundary by more than the 1e-4 band, and the discrete
iteration then follows another path), while every single step still matches the
oracle's map; the W4 pipeline therefore gates the map at every step and reports the
whole run (see layer_parity.admm_rows_trajectory)."""
import numpy as np
import pytest

import qz_synth
from block_driver import run_block, sublayer_names
from gpu_util import qz, report, to_dev, to_host
from layer_parity import (admm_rows_replay, admm_rows_trajectory, check_hessian, gptq_rows,
                          sample_rows)
from oracle import hessian

pytestmark = pytest.mark.gpu

PIPELINES = [(3, "admm"), (4, "gptq")]
STRICT_RUN = {3: True, 4: False}
N_KEEP = 16384
CASES = [(b, m, name) for b, m in PIPELINES for name in sublayer_names()]
_block = {}
_hess = {}


def _run(bits, method):
    key = (bits, method)
    if key not in _block:
        _block.clear()
        _hess.clear()
        _block[key] = run_block(qz(), bits, method, N_KEEP)
    return _block[key]


def _oracle_h(bits, method, rec):
    """Oracle H of a sub-layer's input (fp32 cast), checked once against the GPU build
    of the same tokens."""
    key = (bits, method, rec["input"])
    if key not in _hess:
        n_h = N_KEEP
        Xh = rec["X_head"][:n_h]
        damp = qz_synth.BLOCK_8B["damp"]
        G = hessian.gram(Xh)
        out = qz().qz_build_hessian(to_dev(Xh), damp=damp)
        w = check_hessian(to_host(out["H"]), G, n_h, float(to_host(out["lam"])[0]), damp,
                          to_host(out["diag"]), to_host(out["sigma"]))
        report("block_hessian", input=rec["input"], n=n_h, d=rec["d_i"], worst_over_tol=f"{w:.3g}")
        del out
        H = G + hessian.damping(G, damp) * np.eye(G.shape[0])
        _hess.clear()
        _hess[key] = H.astype(np.float32)
    return _hess[key]


@pytest.mark.parametrize("bits,method,name", CASES)
def test_block_sublayer(bits, method, name):
    res = _run(bits, method)
    rec = res[name]
    B = qz_synth.BLOCK_8B
    Hf = _oracle_h(bits, method, rec)
    rows = sample_rows(rec["d_o"])
    tag = f"{name}_w{bits}_{method}"
    _, f_gptq = gptq_rows(tag, Hf, rec["W"], rows, bits, B["group"], B["B"])
    if rec["d_i"] <= 4096 or STRICT_RUN[bits]:
        admm_rows_trajectory(tag, Hf, rec["W"], rows, bits, B["group"], B["iters"], B["rho0"],
                             B["gamma"], B["refresh"], B=B["B"], strict=STRICT_RUN[bits])
    else:
        T = B["iters"]
        admm_rows_replay(tag, Hf, rec["W"], rows, bits, B["group"], T, B["rho0"], B["gamma"],
                         B["refresh"], [0, T // 2, T - 1], f_gptq=f_gptq)
    # the propagated codes are valid b-bit codes
    assert int(rec["codes"].max()) <= (1 << bits) - 1
