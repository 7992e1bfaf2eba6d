"""Host-side checks of bench.py (no GPU): the one-GPU contract, the algorithmic cost model
and the CPU baseline's record."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from test_sequence_layers_amd.workloads import workload  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in json.loads(p.stdout.strip())["error"]


def test_algorithmic_bytes_and_flops():
    w = workload("linear_d64_T2048")
    b, f = bench.algorithmic_cost(w)
    tok = 8 * 12 * 2048 * 64 * 2
    assert b == 4 * tok + 12 * 64 * 64 * 4             # Q, K, V read, Z written, W0 read
    # per head-token: K W^T, Q W^T, the update (3 x 2 d^2) and the two b x d tril products
    assert f == 8 * 12 * 2048 * (6 * 64 * 64 + 2 * 16 * 64)
    m = workload("mlp_h256_T2048")
    _, fm = bench.algorithmic_cost(m)
    assert fm == 8 * 12 * 2048 * (14 * 64 * 256 + 2 * 16 * (64 + 256))
    d = workload("delta_d64_T8192")
    bd, fd = bench.algorithmic_cost(d)
    assert bd == 4 * 4 * 16 * 8192 * 64 * 2 + 16 * 64 * 64 * 4
    assert fd == 4 * 16 * 8192 * 6 * 64 * 64          # token by token, no chunk products


def test_cpu_baseline_record():
    w = workload("linear_d64_T2048").replace(B=1, H=2, T=64)
    r = bench.cpu_baseline(w, budget_s=0.02, repeats=1)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] >= 1 and r["one_thread"]["cores"] == 1 and r["float64"]["value"] > 0
    assert "sequences" in r["sample"] and r["cpu_model"]
