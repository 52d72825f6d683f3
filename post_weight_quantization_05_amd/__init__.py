"""Python binding of libqz, the gfx950 HIP library behind include/qz.h.

Argument marshalling only: tensors are allocated with PyTorch on the current CUDA
(HIP) device, their pointers and the current stream are passed through ctypes, and
every step of every solver runs in the library's kernels.  The functions carry the
C names; see include/qz.h for the operation each one performs and its citation.

Importing this package does not load the library; the first call does, and fails
loudly if libqz.so has not been built (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import (QZ_ADMM_DUAL_NO_RESCALE, QZ_ADMM_REFRESH_FROM_Z, QZ_ADMM_REFRESH_UNCLAMPED,  # noqa: F401
                   QZ_ADMM_WARM_START, QZ_BF16, QZ_F32, QZ_GRID_CALLER, QZ_H_ACCUMULATE,
                   QZ_H_NO_FINALIZE, QzAdmm, QzGrid)


class QzError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {message}")


def lib():
    return _lib.load()


def _check(status: int):
    if status != 0:
        raise QzError(status, lib().qz_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.QZ_BF16
    if t.dtype == torch.float32:
        return _lib.QZ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _grid(bits, group, caller=False):
    return QzGrid(C.sizeof(QzGrid), int(bits), int(group), _lib.QZ_GRID_CALLER if caller else 0)


def _workspace(nbytes, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def qz_abi_version() -> int:
    return lib().qz_abi_version()


def qz_hessian_workspace(n, d_i, xt=_lib.QZ_BF16) -> int:
    return lib().qz_hessian_workspace(n, d_i, xt)


def qz_build_hessian(X, damp=0.01, flags=0, H=None, ws=None, scaled=False):
    """H = X^T X + lambda I (X [n x d_i] bf16 or fp32 on the GPU).  Returns
    dict(H, diag, sigma, lam, H_scaled) (tensors; lam is a 1-element tensor; H_scaled =
    Sigma H Sigma when scaled=True, else None)."""
    torch = _torch()
    _dev(X, "X")
    n, d = X.shape
    xt = _dtype_code(X)
    dev = X.device
    if H is None:
        H = torch.empty((d, d), dtype=torch.float32, device=dev)
    diag = torch.empty(d, dtype=torch.float32, device=dev)
    sigma = torch.empty(d, dtype=torch.float32, device=dev)
    lam = torch.empty(1, dtype=torch.float32, device=dev)
    Hs = torch.empty((d, d), dtype=torch.float32, device=dev) if scaled else None
    need = lib().qz_hessian_workspace(n, d, xt)
    if ws is None:
        ws = _workspace(need, dev)
    _check(lib().qz_build_hessian(_ptr(X), xt, n, d, float(damp), int(flags), _ptr(H), _ptr(diag),
                                  _ptr(sigma), _ptr(Hs), _ptr(lam), _ptr(ws), ws.numel(),
                                  _stream()))
    return dict(H=H, diag=diag, sigma=sigma, lam=lam, H_scaled=Hs)


def qz_rtn_workspace(d_o, d_i) -> int:
    return lib().qz_rtn_workspace(d_o, d_i)


def qz_rtn(W, bits, group, scales=None, zeros=None, ws=None):
    """Round-to-nearest codes on the grid fit from W (or the given grid)."""
    torch = _torch()
    _dev(W, "W")
    d_o, d_i = W.shape
    caller = scales is not None
    G = d_i // group if group > 0 and d_i % group == 0 else 0
    if not caller:
        scales = torch.empty((d_o, G), dtype=torch.float32, device=W.device)
        zeros = torch.empty((d_o, G), dtype=torch.uint8, device=W.device)
    codes = torch.empty((d_o, d_i), dtype=torch.uint8, device=W.device)
    if ws is None:
        ws = _workspace(lib().qz_rtn_workspace(d_o, d_i), W.device)
    g = _grid(bits, group, caller)
    _check(lib().qz_rtn(_ptr(W), _dtype_code(W), d_o, d_i, C.byref(g), _ptr(codes), _ptr(scales),
                        _ptr(zeros), _ptr(ws), ws.numel(), _stream()))
    return codes, scales, zeros


def qz_rtn_noalloc(W, bits, group, scales=None, zeros=None, codes=None):
    """qz_rtn without a workspace (the library's static per-GPU status word; calls that
    overlap on one GPU race on it).  Outputs may be passed in so that nothing is
    allocated here either."""
    torch = _torch()
    _dev(W, "W")
    d_o, d_i = W.shape
    caller = scales is not None
    G = d_i // group if group > 0 and d_i % group == 0 else 0
    if not caller:
        scales = torch.empty((d_o, G), dtype=torch.float32, device=W.device)
        zeros = torch.empty((d_o, G), dtype=torch.uint8, device=W.device)
    if codes is None:
        codes = torch.empty((d_o, d_i), dtype=torch.uint8, device=W.device)
    g = _grid(bits, group, caller)
    _check(lib().qz_rtn_noalloc(_ptr(W), _dtype_code(W), d_o, d_i, C.byref(g), _ptr(codes),
                                _ptr(scales), _ptr(zeros), _stream()))
    return codes, scales, zeros


def qz_gptq_workspace(d_o, d_i, B) -> int:
    return lib().qz_gptq_workspace(d_o, d_i, B)


def qz_gptq(H, W_hat, bits, group, B=128, perm=None, scales=None, zeros=None, ws=None):
    """GPTQ codes and grid for W_hat [d_o x d_i] given H [d_i x d_i]."""
    torch = _torch()
    _dev(H, "H")
    _dev(W_hat, "W_hat")
    d_o, d_i = W_hat.shape
    caller = scales is not None
    G = d_i // group if group > 0 and d_i % group == 0 else 0
    if not caller:
        scales = torch.empty((d_o, G), dtype=torch.float32, device=W_hat.device)
        zeros = torch.empty((d_o, G), dtype=torch.uint8, device=W_hat.device)
    codes = torch.empty((d_o, d_i), dtype=torch.uint8, device=W_hat.device)
    if perm is not None:
        perm = _dev(perm.to(torch.int32), "perm")
    if ws is None:
        ws = _workspace(lib().qz_gptq_workspace(d_o, d_i, B), W_hat.device)
    g = _grid(bits, group, caller)
    _check(lib().qz_gptq(_ptr(H), _ptr(W_hat), _dtype_code(W_hat), d_o, d_i, C.byref(g), int(B),
                         _ptr(perm), _ptr(codes), _ptr(scales), _ptr(zeros), _ptr(ws), ws.numel(),
                         _stream()))
    return codes, scales, zeros


def qz_gptq_noclip(H, W_hat, bits, group, B=128, perm=None, scales=None, zeros=None, ws=None):
    """GPTQ without clipping: int32 codes (may leave [0, 2^bits - 1]) and the grid."""
    torch = _torch()
    _dev(H, "H")
    _dev(W_hat, "W_hat")
    d_o, d_i = W_hat.shape
    caller = scales is not None
    G = d_i // group if group > 0 and d_i % group == 0 else 0
    if not caller:
        scales = torch.empty((d_o, G), dtype=torch.float32, device=W_hat.device)
        zeros = torch.empty((d_o, G), dtype=torch.uint8, device=W_hat.device)
    codes = torch.empty((d_o, d_i), dtype=torch.int32, device=W_hat.device)
    if perm is not None:
        perm = _dev(perm.to(torch.int32), "perm")
    if ws is None:
        ws = _workspace(lib().qz_gptq_workspace(d_o, d_i, B), W_hat.device)
    g = _grid(bits, group, caller)
    _check(lib().qz_gptq_noclip(_ptr(H), _ptr(W_hat), _dtype_code(W_hat), d_o, d_i, C.byref(g),
                                int(B), _ptr(perm), _ptr(codes), _ptr(scales), _ptr(zeros),
                                _ptr(ws), ws.numel(), _stream()))
    return codes, scales, zeros


def qz_order(H, kind, pivots=False, ws=None):
    """Quantization order for qz_gptq's perm: kind "act" or "min_pivot".  Returns perm
    (int32) or, with pivots=True (min_pivot only), (perm, LDL pivots fp64)."""
    torch = _torch()
    _dev(H, "H")
    d = H.shape[0]
    k = {"act": _lib.QZ_ORDER_ACT, "min_pivot": _lib.QZ_ORDER_MIN_PIVOT}[kind]
    perm = torch.empty(d, dtype=torch.int32, device=H.device)
    piv = torch.empty(d, dtype=torch.float64, device=H.device) if pivots else None
    if ws is None:
        ws = _workspace(lib().qz_order_workspace(d, k), H.device)
    _check(lib().qz_order(_ptr(H), d, k, _ptr(perm), _ptr(piv), _ptr(ws), ws.numel(), _stream()))
    return (perm, piv) if pivots else perm


def qz_error_bound(H, scales, group, perm=None, rows=False, ws=None):
    """Theorem 5 bound on the no-clip layer objective in order perm: the total (float)
    and, with rows=True, the per-row bounds (device fp64)."""
    torch = _torch()
    _dev(H, "H")
    _dev(scales, "scales")
    d_i = H.shape[0]
    d_o = scales.shape[0]
    if perm is not None:
        perm = _dev(perm.to(torch.int32), "perm")
    out = C.c_double(0.0)
    rb = torch.empty(max(d_o, 1), dtype=torch.float64, device=H.device)
    if ws is None:
        ws = _workspace(lib().qz_error_bound_workspace(d_o, d_i), H.device)
    _check(lib().qz_error_bound(_ptr(H), d_i, _ptr(perm), _ptr(scales), d_o, int(group), _ptr(rb),
                                C.byref(out), _ptr(ws), ws.numel(), _stream()))
    return (out.value, rb[:d_o]) if rows else out.value


def qz_admmq_prepare_workspace(d_i) -> int:
    return lib().qz_admmq_prepare_workspace(d_i)


def qz_admmq_prepare(H, ws=None):
    """(V, Lambda, sigma) with Sigma H Sigma = V diag(Lambda) V^T."""
    torch = _torch()
    _dev(H, "H")
    d = H.shape[0]
    V = torch.empty((d, d), dtype=torch.float32, device=H.device)
    lam = torch.empty(d, dtype=torch.float32, device=H.device)
    sigma = torch.empty(d, dtype=torch.float32, device=H.device)
    if ws is None:
        need = lib().qz_admmq_prepare_workspace(d)
        if need == 0:
            _check(-5)
        ws = _workspace(need, H.device)
    _check(lib().qz_admmq_prepare(_ptr(H), d, _ptr(V), _ptr(lam), _ptr(sigma), _ptr(ws), ws.numel(),
                                  _stream()))
    return V, lam, sigma


def qz_admmq_workspace(d_o, d_i, group, iters) -> int:
    return lib().qz_admmq_workspace(d_o, d_i, group, iters)


def qz_admmq(V, Lambda, sigma, W_hat, bits, group, iters, rho0, gamma, refresh_every=1, flags=0,
             t0=0, state=None, scales=None, zeros=None, ws=None, want_U=True):
    """ADMM-Q.  state: dict(codes, scales, zeros, U) to resume (sets QZ_ADMM_WARM_START;
    the tensors are updated in place).  Returns dict(codes, scales, zeros, U, residuals)."""
    torch = _torch()
    for t, nm in ((V, "V"), (Lambda, "Lambda"), (sigma, "sigma"), (W_hat, "W_hat")):
        _dev(t, nm)
    d_o, d_i = W_hat.shape
    dev = W_hat.device
    G = d_i // group if group > 0 and d_i % group == 0 else 0
    caller = scales is not None
    if state is not None:
        flags |= _lib.QZ_ADMM_WARM_START
        codes, scales, zeros, U = state["codes"], state["scales"], state["zeros"], state["U"]
    else:
        codes = torch.empty((d_o, d_i), dtype=torch.uint8, device=dev)
        if not caller:
            scales = torch.empty((d_o, G), dtype=torch.float32, device=dev)
            zeros = torch.empty((d_o, G), dtype=torch.uint8, device=dev)
        U = torch.empty((d_o, d_i), dtype=torch.float32, device=dev) if want_U else None
    res = torch.empty((max(iters, 1), 2), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib().qz_admmq_workspace(d_o, d_i, group, iters), dev)
    g = _grid(bits, group, caller)
    p = QzAdmm(C.sizeof(QzAdmm), int(iters), float(rho0), float(gamma), int(refresh_every), int(flags),
               int(t0))
    _check(lib().qz_admmq(_ptr(V), _ptr(Lambda), _ptr(sigma), _ptr(W_hat), _dtype_code(W_hat), d_o,
                          d_i, C.byref(g), C.byref(p), _ptr(codes), _ptr(scales), _ptr(zeros),
                          _ptr(U), _ptr(res), _ptr(ws), ws.numel(), _stream()))
    return dict(codes=codes, scales=scales, zeros=zeros, U=U, residuals=res[:iters])


def qz_objective_workspace(d_o, d_i) -> int:
    return lib().qz_objective_workspace(d_o, d_i)


def qz_objective(H, W_hat, codes, scales, zeros, group, rows=False, ws=None):
    """f = 1/2 sum_r (q_r - w_r)^T H (q_r - w_r) for q = s (codes - z), codes uint8 or int32
    (no-clip GPTQ).  Returns the float (and, with rows=True, the per-row fp64 objectives as
    a device tensor)."""
    torch = _torch()
    for t, nm in ((H, "H"), (W_hat, "W_hat"), (codes, "codes"), (scales, "scales"), (zeros, "zeros")):
        _dev(t, nm)
    d_o, d_i = W_hat.shape
    if ws is None:
        ws = _workspace(lib().qz_objective_workspace(d_o, d_i), W_hat.device)
    row_f = torch.empty(d_o, dtype=torch.float64, device=W_hat.device) if rows else None
    out = C.c_double(0.0)
    fn = lib().qz_objective_i32 if codes.dtype == torch.int32 else lib().qz_objective
    _check(fn(_ptr(H), _ptr(W_hat), _dtype_code(W_hat), _ptr(codes), _ptr(scales), _ptr(zeros), d_o,
              d_i, int(group), _ptr(row_f), C.byref(out), _ptr(ws), ws.numel(), _stream()))
    return (out.value, row_f) if rows else out.value


def qz_local_search_workspace(d_o, d_i, group) -> int:
    return lib().qz_local_search_workspace(d_o, d_i, group)


def qz_local_search(H, W_hat, codes, scales, zeros, bits, group, max_steps, ws=None):
    """Pairwise-swap local search on the fixed grid; codes are updated in place.
    Returns (steps that moved, [moves accepted per step])."""
    for t, nm in ((H, "H"), (W_hat, "W_hat"), (codes, "codes"), (scales, "scales"), (zeros, "zeros")):
        _dev(t, nm)
    d_o, d_i = W_hat.shape
    if ws is None:
        ws = _workspace(lib().qz_local_search_workspace(d_o, d_i, group), W_hat.device)
    moves = (C.c_int32 * max(int(max_steps), 1))()
    steps = C.c_int32(0)
    g = _grid(bits, group, True)
    _check(lib().qz_local_search(_ptr(H), _ptr(W_hat), _dtype_code(W_hat), d_o, d_i, C.byref(g),
                                 _ptr(scales), _ptr(zeros), _ptr(codes), int(max_steps), moves,
                                 C.byref(steps), _ptr(ws), ws.numel(), _stream()))
    return steps.value, list(moves)[:steps.value + (1 if steps.value < max_steps else 0)]


def qz_packed_words(cols, bits) -> int:
    return lib().qz_packed_words(cols, bits)


def qz_pack(codes, bits):
    torch = _torch()
    _dev(codes, "codes")
    rows, cols = codes.shape
    out = torch.empty((rows, max(lib().qz_packed_words(cols, bits), 0)), dtype=torch.int32,
                      device=codes.device)
    _check(lib().qz_pack(_ptr(codes), rows, cols, int(bits), _ptr(out), _stream()))
    return out


def qz_unpack(words, cols, bits):
    torch = _torch()
    _dev(words, "words")
    rows = words.shape[0]
    out = torch.empty((rows, cols), dtype=torch.uint8, device=words.device)
    _check(lib().qz_unpack(_ptr(words), rows, cols, int(bits), _ptr(out), _stream()))
    return out


def qz_timing_enable(on=True):
    _check(lib().qz_timing_enable(1 if on else 0))


def qz_timing_read(reset=True):
    """{kind name: (launches, total_ms)} of the launches recorded while timing was on."""
    n = 32
    launches = (C.c_int64 * n)()
    total = (C.c_double * n)()
    k = lib().qz_timing_read(launches, total, n, 1 if reset else 0)
    if k < 0:
        _check(k)
    return {lib().qz_timing_kind_name(i).decode(): (launches[i], total[i]) for i in range(min(k, n))
            if launches[i] > 0}


def qz_last_error() -> str:
    return lib().qz_last_error().decode(errors="replace")
