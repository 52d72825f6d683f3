"""CPU checks of bench.py's contract: one GPU only, the measured traffic it reports belongs
to the current kernel sources, and the algorithmic work per launch it divides by.  Nothing
here touches a GPU."""
import os
import subprocess
import sys

import bench
import qz_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_traffic_figures_belong_to_the_current_sources():
    # bench.py reports a kernel's measured HBM bytes only while its source is the one the
    # counters were taken on; every stored figure must still apply to the headline line
    for kind in bench.TRAFFIC:
        assert bench.traffic_bytes(kind, bench.TRAFFIC_WORKLOAD) is not None, kind
    assert bench.traffic_bytes("hessian_gram_bf16", "attn_4096x4096_w3g128") is None
    assert bench.TRAFFIC_WORKLOAD == bench.HEADLINE


def test_gptq_work_matches_hand_counts():
    # 2 blocks of 2 columns on 3 rows: block 0 updates the 2 later columns with K = 2
    # (2 * 3 * 2 * 2 = 24 flops), block 1 has none; in-block updates 3 * 2 * 3 per block
    tr, ib = bench.gptq_work(3, 4, 2)
    assert tr == 24.0 and ib == 36.0
    # a ragged last block of 1 column
    tr, ib = bench.gptq_work(1, 5, 2)
    assert tr == 2 * 2 * 3 + 2 * 2 * 1 and ib == 2 * 3 + 2 * 3 + 1 * 2


def test_headline_workload_is_the_metric_layer():
    cfg = qz_synth.WORKLOADS[bench.HEADLINE]
    assert (cfg["d_i"], cfg["d_o"], cfg["bits"], cfg["group"]) == (4096, 12288, 3, 128)
    assert cfg["n"] == 262144 and cfg["iters"] == 100
    # the per-launch work bench.py divides by, written out for this layer
    assert 2.0 * cfg["d_o"] * cfg["d_i"] ** 2 == 412316860416.0       # one W-update product
    assert 18.0 * cfg["d_o"] * cfg["d_i"] == 905969664.0                # projection bytes
    assert 1.0 * cfg["n"] * cfg["d_i"] * (cfg["d_i"] + 1) == 4399120252928.0   # Hessian
