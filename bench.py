"""Benchmark of the layer quantizer's hot path on one MI355X.

One step = one pass of the whole path over one layer: Hessian build from the
calibration tokens, GPTQ (grid, inverse factor, column loop), ADMM-Q (one-time
eigendecomposition, then the iteration loop) and packing of both results.
Inputs (calibration activations and weights) are synthetic, seeded, and resident in
HBM before the timed region starts.

The headline value is ADMM-Q iterations per second of the loop (set-up and the
eigendecomposition excluded, they are reported separately), next to the GPTQ layer
time and the Hessian TFLOP/s.  Per-kernel durations come from the library's HIP
events (qz_timing_*), recorded on the stream the kernels run on.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import qz_synth  # noqa: E402

METRIC = "ADMM-Q iters/s + GPTQ layer time, 4096×12288 W3g128; H-build TFLOP/s"
HEADLINE = "up_4096x12288_w3g128"

PEAK_BF16 = 2.5e15        # dense MFMA, FLOP/s
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12         # B/s
PEAK_FP32_VALU = 157.3e12  # vector fp32 (packed), FLOP/s
PEAK_FP64 = 78.6e12        # vector / matrix fp64, FLOP/s

# HBM-side bytes per launch on the headline workload, from two rocprofv3 --pmc runs
# (FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0, the factors that make a plain 1 GiB streaming
# kernel read 1 GiB and write 1 GiB; bench.py --copy-probe is that kernel), with the
# SHA-256 of the kernel's source file at the time.  A kernel whose source has changed
# since reports null.
TRAFFIC = {
    "gemm_admm_wupdate1": (5004.4e6, "k_gemm.hip",
                          "4b3b79ff82303147030bf74c271647bb946e67de79935df19ec0b3d93bad1e6a"),
    "gemm_admm_wupdate2": (6754.9e6, "k_gemm.hip",
                          "4b3b79ff82303147030bf74c271647bb946e67de79935df19ec0b3d93bad1e6a"),
    "admm_project": (932.4e6, "k_admm.hip",
                    "e3f70300b61a47cdee85889e1ec3a8654dbc49310bc60d5cd8d2f4e4b4851f12"),
    "hessian_gram_bf16": (14558.0e6, "k_hessian.hip",
                         "2a1ccf1ce62306db32ddea42ac13c0a6dcc82e25da215221220577df49397698"),
}
TRAFFIC_WORKLOAD = "up_4096x12288_w3g128"


def traffic_bytes(kind, workload):
    """Measured HBM bytes per launch, or None (other workload, or the kernel changed)."""
    import hashlib
    if workload != TRAFFIC_WORKLOAD or kind not in TRAFFIC:
        return None
    nbytes, src, digest = TRAFFIC[kind]
    path = os.path.join(ROOT, "post_weight_quantization_05_amd", "csrc", src)
    try:
        with open(path, "rb") as f:
            cur = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return nbytes if cur == digest else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(qz_synth.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=3072)
    ap.add_argument("--cpu-iters", type=int, default=40)
    ap.add_argument("--ls-steps", type=int, default=256,
                    help="step limit of the local search run on ADMM-Q's result (outside the timed steps)")
    ap.add_argument("--sweep", action="store_true",
                    help="one line per layer workload (1 warm-up and 1 timed step each), no CPU, "
                         "orders or local-search legs")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain streaming kernel (y = -x over MIB MiB of fp32, 3 launches) "
                         "whose byte counts calibrate the HBM traffic counters, then exit")
    return ap.parse_args()


def copy_probe(mib):
    """A kernel of known traffic: each launch reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 3}), flush=True)


def _host_info():
    """CPU model and the BLAS library NumPy runs on, with its thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:  # noqa: BLE001
        pass
    return model, blas, int(threads)


def cpu_baseline(cfg, X, W_bits, rows, iters, gptq_rows=1024):
    """The fp64 oracle on the host: ADMM-Q iterations on a sample of rows (rows are
    independent), scaled to the whole layer; the eigendecomposition is excluded from
    the value as it is on the GPU, and timed as a phase.  H comes from the oracle on the
    same tokens.  Phases also time GPTQ's inverse factor and its column loop on a smaller
    row sample (scaled to the layer)."""
    import numpy as np
    from oracle import admm, gptq, grid, hessian
    model, blas, cores = _host_info()
    n_sample = min(X.shape[0], 16384)
    Xs = X[:n_sample]
    t0 = time.perf_counter()
    H, _ = hessian.hessian(Xs, cfg["damp"])
    t_h = time.perf_counter() - t0
    t0 = time.perf_counter()
    spec = admm.spectral(H)
    t_eig = time.perf_counter() - t0
    Wf = qz_synth.bf16_bits_to_f32(W_bits[:rows])
    t0 = time.perf_counter()
    admm.admm(H, Wf, cfg["bits"], cfg["group"], iters, cfg["rho0"], cfg["gamma"], cfg["refresh"],
              spec=spec)
    t_loop = time.perf_counter() - t0
    per_iter_layer = t_loop / iters * (cfg["d_o"] / rows)
    t0 = time.perf_counter()
    R = gptq.inverse_factor_lapack(H)
    t_r = time.perf_counter() - t0
    g = min(gptq_rows, rows)
    s_, z_ = grid.fit_grid_f32(Wf[:g], cfg["bits"], cfg["group"])
    t0 = time.perf_counter()
    gptq.gptq(None, Wf[:g], s_, z_, cfg["bits"], cfg["group"], R=R)
    t_gl = time.perf_counter() - t0
    return {"value": 1.0 / per_iter_layer, "unit": "iters/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {cfg['d_o']} rows x {iters} ADMM iterations (fp64 NumPy, H from "
                      f"{n_sample} tokens, eigendecomposition excluded), scaled to the full layer; "
                      f"loop {t_loop:.2f} s, H build {t_h:.2f} s",
            "cpu": model, "blas": blas,
            "phases_s": {"hessian_16384_tokens": round(t_h, 3), "eigendecomposition": round(t_eig, 3),
                         "admm_per_iteration_layer": round(per_iter_layer, 3),
                         "gptq_inverse_factor": round(t_r, 3),
                         "gptq_loop_layer": round(t_gl * cfg["d_o"] / g, 3),
                         "gptq_rows_timed": g}}


def gptq_work(d_o, d_i, B):
    """flops of the GPTQ loop: the trailing products W[:, b:] -= E R[a:b, b:] summed over
    blocks, and the in-block column updates."""
    trailing, inblock = 0.0, 0.0
    for a in range(0, d_i, B):
        b = min(a + B, d_i)
        trailing += 2.0 * d_o * (b - a) * (d_i - b)
        inblock += 1.0 * d_o * (b - a) * (b - a + 1)
    return trailing, inblock


def run_workload(args, name, steps, warmup, with_cpu, legs=True):
    """One bench line for workload `name` (inputs resident in HBM before timing)."""
    import numpy as np
    import torch
    import post_weight_quantization_05_amd as q

    cfg = dict(qz_synth.WORKLOADS[name])
    d_i, d_o, n = cfg["d_i"], cfg["d_o"], cfg["n"]
    bits, group, B, iters = cfg["bits"], cfg["group"], cfg["B"], cfg["iters"]
    seed = cfg.get("seed", 1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs resident in HBM
    X = qz_synth.calib_bf16_torch(seed, n, d_i, cfg["p_out"], cfg["f_out"], device=dev)
    W = qz_synth.weights_bf16_torch(seed, d_o, d_i, device=dev)
    H = torch.empty((d_i, d_i), dtype=torch.float32, device=dev)
    ws_h = torch.empty(max(q.qz_hessian_workspace(n, d_i), 1), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(q.qz_gptq_workspace(d_o, d_i, B), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(q.qz_admmq_workspace(d_o, d_i, group, iters), dtype=torch.uint8, device=dev)
    ws_e = torch.empty(q.qz_admmq_prepare_workspace(d_i), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(record):
        e = [ev() for _ in range(7)]
        e[0].record(stream)
        hb = q.qz_build_hessian(X, damp=cfg["damp"], H=H, ws=ws_h)
        e[1].record(stream)
        gc, gs, gz = q.qz_gptq(hb["H"], W, bits, group, B, ws=ws_g)
        e[2].record(stream)
        gp = q.qz_pack(gc, bits)
        e[3].record(stream)
        V, lam, sig = q.qz_admmq_prepare(hb["H"], ws=ws_e)
        e[4].record(stream)
        out = q.qz_admmq(V, lam, sig, W, bits, group, iters, cfg["rho0"], cfg["gamma"],
                         cfg["refresh"], ws=ws_a, want_U=False)
        e[5].record(stream)
        ap = q.qz_pack(out["codes"], bits)
        e[6].record(stream)
        if record is not None:
            record.append((e, out["residuals"]))
        return gp, ap

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()

    # the timed steps run without the library's per-launch timers (whose event records
    # would sit between the kernels); one more step, untimed, collects the per-kernel times
    recs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q.qz_timing_read(reset=True)
    q.qz_timing_enable(True)
    step(None)
    torch.cuda.synchronize()
    q.qz_timing_enable(False)
    kt = q.qz_timing_read(reset=True)

    # ---- per-phase times (ms) from the events
    ph = {k: [] for k in ("hbuild", "gptq", "pack_gptq", "admm_prepare", "admm", "pack_admm")}
    for e, _ in recs:
        vals = [e[i].elapsed_time(e[i + 1]) for i in range(6)]
        for k, v in zip(ph, vals):
            ph[k].append(v)
    med = {k: float(np.median(v)) for k, v in ph.items()}
    kn = {k: v for k, v in kt.items()}
    loop_kinds = ("gemm_admm_wupdate1", "gemm_admm_wupdate2", "admm_project")
    admm_loop_ms = sum(kn[k][1] for k in loop_kinds if k in kn)   # the one instrumented step
    admm_call_ms = med["admm"]
    iters_per_s = iters / (admm_call_ms / 1e3)
    iters_per_s_loop = iters / (admm_loop_ms / 1e3) if admm_loop_ms > 0 else None

    # ---- rooflines (algorithmic work per launch / average launch duration)
    def avg_ms(kind):
        c, t = kn.get(kind, (0, 0.0))
        return t / c if c else None

    gemm_flops = 2.0 * d_o * d_i * d_i                      # one W-update product
    proj_bytes = 18.0 * d_o * d_i                           # read W~,U,C_old; write U,M,C
    hb_flops = 1.0 * n * d_i * (d_i + 1)                    # upper triangle of X^T X
    gemm1_bytes = 4.0 * (2 * d_o * d_i + d_i * d_i + d_o * d_i)   # read M, P, V; write T
    gemm2_bytes = 4.0 * (d_o * d_i + d_i * d_i + d_o * d_i)       # read T, V; write W~
    tr_flops, ib_flops = gptq_work(d_o, d_i, B)
    n_blocks = -(-d_i // B)
    pack_bytes = d_o * d_i * (1.0 + bits / 8.0)
    # per launch: the trailing product and the block kernel run once per block (the
    # last block has no trailing product); the R factor and packing once per layer
    rows = (
        ("gemm_admm_wupdate1", gemm_flops, PEAK_FP32_MFMA, "mfma", "TFLOP/s", gemm1_bytes),
        ("gemm_admm_wupdate2", gemm_flops, PEAK_FP32_MFMA, "mfma", "TFLOP/s", gemm2_bytes),
        ("admm_project", proj_bytes, PEAK_HBM, "hbm", "GB/s", proj_bytes),
        ("hessian_gram_bf16", hb_flops, PEAK_BF16, "mfma", "TFLOP/s", 2.0 * n * d_i),
        ("gemm_gptq_trailing", tr_flops / max(n_blocks - 1, 1), PEAK_FP32_MFMA, "mfma", "TFLOP/s", None),
        ("gptq_block", ib_flops / n_blocks, PEAK_FP32_VALU, "alu", "TFLOP/s", None),
        ("rfactor_fp64", 2.0 / 3.0 * d_i ** 3, PEAK_FP64, "alu", "TFLOP/s", None),
        ("pack", pack_bytes, PEAK_HBM, "hbm", "GB/s", pack_bytes),
    )
    rl = []
    for kind, work, peak, bound, unit, alg in rows:
        a = avg_ms(kind)
        if a is None:
            continue
        rate = work / (a / 1e3)
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        rl.append({"kernel": kind, "bound": bound, "achieved": round(rate / scale, 3),
                   "peak": round(peak / scale, 3), "unit": unit, "frac": round(rate / peak, 4),
                   "avg_ms": round(a, 4), "launches": kn[kind][0],
                   "traffic": traffic_bytes(kind, name),
                   "traffic_unit": "B/launch", "algorithmic_bytes": alg})
    dominant = max((r for r in rl if r["kernel"].startswith("gemm_admm")),
                   key=lambda r: r["avg_ms"] * r["launches"], default=None)

    res_last = recs[-1][1][-1].tolist() if recs else None
    gptq_ms = med["gptq"]
    # ---- layer-level rooflines: the time each solver would take with every kernel at its
    # peak (matrix-core products at the fp32 MFMA peak, the fp64 factor at the fp64 peak,
    # streaming at the HBM peak), against the measured time of the whole call
    it_roof_s = 4.0 * d_o * d_i * d_i / PEAK_FP32_MFMA + proj_bytes / PEAK_HBM
    admm_setup_roof_s = 2.0 * d_o * d_i * d_i / PEAK_FP32_MFMA      # P = W~_hat V Lambda
    admm_roof_ms = (iters * it_roof_s + admm_setup_roof_s) * 1e3
    gptq_roof_ms = (tr_flops / PEAK_FP32_MFMA + 2.0 / 3.0 * d_i ** 3 / PEAK_FP64) * 1e3
    hb_roof_ms = hb_flops / PEAK_BF16 * 1e3
    layer_rl = {
        "admm_iters_per_s": {"achieved": round(iters_per_s, 3),
                             "roofline": round(1.0 / it_roof_s, 3),
                             "frac": round(iters_per_s * it_roof_s, 4),
                             "roofline_basis": "4 d_o d_i^2 flops at the fp32 MFMA peak + 18 B per "
                                               "weight at the HBM peak, per iteration"},
        "admm_weights_per_s": {"achieved": round(d_o * d_i / (admm_call_ms / 1e3), 1),
                               "roofline": round(d_o * d_i / (admm_roof_ms / 1e3), 1),
                               "frac": round(admm_roof_ms / admm_call_ms, 4),
                               "roofline_basis": "set-up product + iterations at their peaks; the "
                                                 "eigendecomposition (a library call) is excluded "
                                                 "on both sides"},
        "gptq_weights_per_s": {"achieved": round(d_o * d_i / (gptq_ms / 1e3), 1),
                               "roofline": round(d_o * d_i / (gptq_roof_ms / 1e3), 1),
                               "frac": round(gptq_roof_ms / gptq_ms, 4),
                               "layer_ms": round(gptq_ms, 3), "roofline_ms": round(gptq_roof_ms, 3),
                               "roofline_basis": "trailing products at the fp32 MFMA peak + 2/3 d_i^3 "
                                                 "at the fp64 peak (the in-block loop is not credited)"},
        "hbuild_tflops": {"achieved": round(hb_flops / (med["hbuild"] / 1e3) / 1e12, 3),
                          "roofline": round(PEAK_BF16 / 1e12, 3),
                          "frac": round(hb_roof_ms / med["hbuild"], 4),
                          "roofline_basis": "n d_i (d_i + 1) flops (upper triangle) at the bf16 "
                                            "MFMA peak, whole call"},
    }
    line = {
        "metric": METRIC,
        "value": round(iters_per_s, 3),
        "unit": "iters/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "d_i": d_i, "d_o": d_o, "bits": bits, "group": group,
                   "n_tokens": n, "gptq_block": B, "admm_iters": iters, "rho0": cfg["rho0"],
                   "gamma": cfg["gamma"], "refresh_every": cfg["refresh"],
                   "global_batch": n, "parallelism": "single-gpu"},
        "components": {
            "admm_iters_per_s": round(iters_per_s, 3),
            "admm_iters_per_s_kernels_only": None if iters_per_s_loop is None else round(iters_per_s_loop, 3),
            "admm_call_ms": round(admm_call_ms, 3),
            "admm_prepare_ms": round(med["admm_prepare"], 3),
            "admm_weights_per_s": round(d_o * d_i / ((admm_call_ms + med["admm_prepare"]) / 1e3), 1),
            "gptq_layer_ms": round(gptq_ms, 3),
            "gptq_weights_per_s": round(d_o * d_i / (gptq_ms / 1e3), 1),
            "gptq_rfactor_ms": round(avg_ms("rfactor_fp64") or 0.0, 3),
            "hbuild_ms": round(med["hbuild"], 3),
            "hbuild_tflops": round(hb_flops / (med["hbuild"] / 1e3) / 1e12, 3),
            "pack_ms": round(med["pack_gptq"] + med["pack_admm"], 4),
            "admm_final_residuals": res_last,
            "kernel_ms": {k: [v[0], round(v[1] / max(v[0], 1), 4)] for k, v in kn.items()},
        },
        "layer_rooflines": layer_rl,
        "rooflines": rl,
        "roofline": None if dominant is None else {k: dominant[k] for k in
                                                   ("bound", "achieved", "peak", "unit", "frac",
                                                    "traffic", "traffic_unit", "algorithmic_bytes",
                                                    "kernel")},
    }
    # layer objective of both results on the full-token H (outside the timed steps)
    gc, gs, gz = q.qz_gptq(H, W, bits, group, B, ws=ws_g)
    f_gptq = q.qz_objective(H, W, gc, gs, gz, group)
    V, lam, sig = q.qz_admmq_prepare(H)
    ao = q.qz_admmq(V, lam, sig, W, bits, group, iters, cfg["rho0"], cfg["gamma"], cfg["refresh"],
                    ws=ws_a, want_U=False)
    f_admm = q.qz_objective(H, W, ao["codes"], ao["scales"], ao["zeros"], group)
    cr, cs, cz = q.qz_rtn(W, bits, group)
    f_rtn = q.qz_objective(H, W, cr, cs, cz, group)
    del V, lam, sig
    line["components"]["objective"] = {"rtn": f_rtn, "gptq": f_gptq, "admmq": f_admm,
                                       "admmq_over_gptq": round(f_admm / f_gptq, 4)}
    if legs:
        line["components"]["local_search"] = local_search_leg(q, H, W, ao, bits, group, f_admm,
                                                              f_gptq, args.ls_steps)
        line["components"]["orders"] = orders_leg(q, H, W, bits, group, B)
        go = {"codes": gc, "scales": gs, "zeros": gz}
        line["components"]["local_search_on_gptq"] = local_search_leg(q, H, W, go, bits, group,
                                                                      f_gptq, f_gptq, args.ls_steps)
        del go
    del ao
    if with_cpu:
        Xh = X[:16384].view(torch.int16).cpu().numpy().view(np.uint16)
        Wh = W[:args.cpu_rows].view(torch.int16).cpu().numpy().view(np.uint16)
        line["cpu_baseline"] = cpu_baseline(cfg, Xh, Wh, args.cpu_rows, args.cpu_iters)
    del X, W, H, ws_h, ws_g, ws_a, ws_e
    torch.cuda.empty_cache()
    return line


def local_search_leg(q, H, W, start, bits, group, f_start, f_gptq, max_steps):
    """Pairwise-swap local search on a solver's result `start` ({"codes", "scales",
    "zeros"}, objective f_start), outside the timed steps: steps, moves per step, time per
    kernel kind and the objective it reaches, relative to the start and to GPTQ's."""
    import torch
    d_o, d_i = W.shape
    ws = torch.empty(q.qz_local_search_workspace(d_o, d_i, group), dtype=torch.uint8,
                     device=W.device)
    codes = start["codes"].clone()
    q.qz_timing_read(reset=True)
    q.qz_timing_enable(True)
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.record()
    steps, moves = q.qz_local_search(H, W, codes, start["scales"], start["zeros"], bits, group,
                                     max_steps, ws=ws)
    e.record()
    torch.cuda.synchronize()
    q.qz_timing_enable(False)
    kt = q.qz_timing_read(reset=True)
    f_ls = q.qz_objective(H, W, codes, start["scales"], start["zeros"], group)
    out = {"steps": steps, "max_steps": max_steps, "moves_per_step": moves,
           "call_ms": round(b.elapsed_time(e), 3),
           "kernel_ms": {k: [v[0], round(v[1] / max(v[0], 1), 4)] for k, v in kt.items()
                         if k.startswith("ls_")},
           "f_after": f_ls, "after_over_start": round(f_ls / f_start, 5),
           "after_over_gptq": round(f_ls / f_gptq, 5)}
    del ws, codes
    return out


def orders_leg(q, H, W, bits, group, B):
    """Quantization orders (outside the timed steps): time of each order, and per order
    (natural, act, min-pivot) the Theorem 5 bound on the no-clip objective, GPTQ's
    objective without clipping and with it."""
    import torch
    out = {}
    perms = {"natural": None}
    for kind in ("act", "min_pivot"):
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        perms[kind] = q.qz_order(H, kind)
        e.record()
        torch.cuda.synchronize()
        out[f"{kind}_order_ms"] = round(b.elapsed_time(e), 3)
    for kind, perm in perms.items():
        cn, sn, zn = q.qz_gptq_noclip(H, W, bits, group, B, perm=perm)
        f_noclip = q.qz_objective(H, W, cn, sn, zn, group)
        bound = q.qz_error_bound(H, sn, group, perm=perm)
        off = float(((cn < 0) | (cn > (1 << bits) - 1)).float().mean().item())
        del cn
        cg, sg, zg = q.qz_gptq(H, W, bits, group, B, perm=perm)
        f_clip = q.qz_objective(H, W, cg, sg, zg, group)
        del cg, sg, zg, sn, zn
        out[kind] = {"bound": bound, "gptq_noclip": f_noclip, "noclip_over_bound": round(f_noclip / bound, 4),
                     "noclip_off_grid": round(off, 5), "gptq": f_clip}
    return out


SWEEP = ("attn_4096x4096_w3g128", "up_4096x12288_w3g128", "mlp_up_4096x12288_w2g128",
         "mlp_down_12288x4096_w2g128", "32b_up_5120x25600_w3g128", "32b_down_25600x5120_w3g128")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the quantizer's rows shard "
              f"across GPUs without per-iteration exchange, but no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.sweep:
        # one line per layer workload (the tiny layer excluded), one timed step each; the
        # orders and local-search legs run on the headline line only
        for name in SWEEP:
            line = run_workload(args, name, 1, 1, False, legs=False)
            line["sweep"] = True
            print(json.dumps(line), flush=True)
        return
    line = run_workload(args, args.workload, args.steps, args.warmup, not args.no_cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
