"""bench.py's accounting, without a GPU.

The roofline numerator (algorithmic bytes and FLOP per stage) is checked
against the per-kernel work table written independently for the layer's
configurations (DeepSeek-V3 prefill, T = 8192: dispatch 1.057 GB, grouped
FFN 5.77 TFLOP and 24.97 GB, combine 1.057 GB; GPT-OSS fp8, T = 4096:
dispatch 72.3 MB, grouped FFN 0.815 TFLOP and about 3.52 GB, combine
118 MB), computed there for balanced routing.  The bound selection and the
one-GPU refusal are checked directly.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def balanced_work(name):
    cfg = wl.CONFIGS[name]
    E_loc = cfg.e_end - cfg.e_begin
    counts = np.full(E_loc, cfg.T * cfg.K // cfg.E, dtype=np.int64)
    work, R, touched = bench.stage_work(cfg, counts, cfg.T)
    return work, R, touched


def test_prefill_work_matches_the_table():
    work, R, touched = balanced_work("dsv3_prefill")
    assert (R, touched) == (65536, 256)
    assert work["dispatch"]["bytes"] / 1e9 == pytest.approx(1.057, abs=5e-4)
    assert work["combine"]["bytes"] / 1e9 == pytest.approx(1.057, abs=5e-4)
    ffn_flops = work["ffn_gate_up"]["flops"] + work["ffn_down"]["flops"]
    ffn_bytes = work["ffn_gate_up"]["bytes"] + work["ffn_down"]["bytes"]
    assert ffn_flops / 1e12 == pytest.approx(5.77, abs=5e-3)
    assert ffn_bytes / 1e9 == pytest.approx(24.97, abs=0.01)   # the table rounds 24.964 up
    # gate/up does two thirds of the FLOP
    assert work["ffn_gate_up"]["flops"] == 2 * work["ffn_down"]["flops"]


def test_gptoss_work_matches_the_table():
    work, R, touched = balanced_work("gptoss_fp8")
    assert (R, touched) == (16384, 128)
    assert work["dispatch"]["bytes"] / 1e6 == pytest.approx(72.3, abs=0.05)
    assert work["combine"]["bytes"] / 1e6 == pytest.approx(118.0, abs=0.2)
    ffn_flops = work["ffn_gate_up"]["flops"] + work["ffn_down"]["flops"]
    ffn_bytes = work["ffn_gate_up"]["bytes"] + work["ffn_down"]["bytes"]
    assert ffn_flops / 1e12 == pytest.approx(0.815, abs=5e-4)
    assert ffn_bytes / 1e9 == pytest.approx(3.52, abs=0.01)


def test_untouched_experts_stream_no_weights():
    cfg = wl.CONFIGS["dsv3_decode"]
    counts = np.zeros(256, dtype=np.int64)
    counts[[3, 17]] = [5, 7]
    work, R, touched = bench.stage_work(cfg, counts, 9)
    assert (R, touched) == (12, 2)
    w_bytes = 2 * 3 * cfg.H * cfg.I * 2          # two experts, three bf16 matrices
    act = R * cfg.H * 2 * 2 + 2 * R * cfg.I * 2  # Xd in, y out, h written and read
    assert work["ffn_gate_up"]["bytes"] + work["ffn_down"]["bytes"] == w_bytes + act


def test_roofline_bound_and_fraction():
    # 8 GB in 1 ms at 1 TFLOP: HBM-bound at exactly the peak
    r = bench.roofline_of({"bytes": 8e9, "flops": 1e12}, 1.0, 2500.0)
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(1.0) and r["unit"] == "GB/s"
    # 1 GB and 2.5 TFLOP in 2 ms: the MFMA floor (1 ms) beats the HBM floor (0.125 ms)
    r = bench.roofline_of({"bytes": 1e9, "flops": 2.5e12}, 2.0, 2500.0)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.5) and r["unit"] == "TFLOP/s"


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
