"""Host-side logic of bench.py (CPU only): algorithmic work, the roofline bound
of the gate/up GEMM per workload, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

import bench
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_flops_of_c3():
    cfg = W.config("c3_qwen3_235b_prefill")
    f, by = bench.algorithmic_work(cfg)
    P = 32768 * 8
    assert f["ffn_gate_up_flop"] == 4.0 * P * 4096 * 1536
    assert f["ffn_down_flop"] == 2.0 * P * 4096 * 1536
    assert f["gate_flop"] == 4.0 * 32768 * 4096 * 128
    # combine: k rows read per token, one row written, 8 bytes of index and weight per pair
    assert by["combine"] == P * 4096 * 2 + 8.0 * P + 32768 * 4096 * 2


@pytest.mark.parametrize("name,active,bound", [("c1_tiny_f32", 16, True), ("c2_qwen3_30b_decode", 80, True),
                                               ("c3_qwen3_235b_prefill", 128, False),
                                               ("c4_glm45_prefill", 160, False), ("c5_olmoe_drift", 64, False)])
def test_gate_up_bound_by_intensity(name, active, bound):
    cfg = W.config(name)
    hbm, achieved, peak, unit, nbytes = bench.gate_up_roofline(cfg, active, 1.0)
    assert hbm == bound
    assert unit == ("GB/s" if bound else "TFLOP/s") and peak == (8000.0 if bound else 2500.0)
    b = cfg.elem_bytes
    assert nbytes == active * 2.0 * cfg.inter * cfg.d * b + cfg.T * cfg.d * b + cfg.P * cfg.inter * b
    # 1 ms: the rate is the work per millisecond
    assert achieved == pytest.approx(nbytes / 1e6 if bound else 4.0 * cfg.P * cfg.d * cfg.inter / 1e9)


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
