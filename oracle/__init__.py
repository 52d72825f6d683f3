"""CPU oracle for the Hessian-weighted layer quantizer (GPTQ and ADMM-Q).

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, deliberately unoptimised
restatement of what the quantizer computes, used to check the GPU library.  Only the
test-suite, the smoke check and the CPU-baseline leg of the benchmark may import it;
the product path never does, and it imports nothing from the product package.

Sources (cited by title and section throughout):

* ADMM-Q page  -- "ADMM-Q: An Improved Hessian-based Weight Quantizer for Post-Training
  Quantization of Large Language Models" (gist.science AI summary, zh/it/ja versions
  agree).  Technical summary, "Methodology": 1. problem formulation; 2. key components
  (diagonal scaling, ADMM splitting with W-update / D-update / dual update, grid
  refresh, local search, convergence under rho_t = rho_0 gamma^t).
* GPTQ tutorial page -- "061 · GPTQ: why the remaining weights compensate the error"
  (wq-win.github.io).  Section 2 (calibration curvature, the Lagrange-multiplier
  compensation, the worked example, damping under collinear channels), section 3
  (Algorithm 1: common column order, blocked lazy update with the upper Cholesky
  factor of the damped inverse curvature), section 4 (128 x 2048 calibration tokens).
* Babai page -- "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
  Algorithm" (gist.science AI summary).  Technical summary 2.1 (CVP, Theorem 1),
  2.2 (Theorem 4, redundancy of composition), 2.3 (Theorem 5 bound, ordering).

Every floating-point step runs in fp64 unless it fixes an fp32 result that the GPU
library must reproduce bit for bit (the grid fit and round-to-nearest, which run in
IEEE fp32 here, see oracle.grid).

Functions whose results have no independent pin say "parity unpinned" in their
docstring.
"""
from . import grid, pack, hessian, gptq, admm, lattice, objective  # noqa: F401
