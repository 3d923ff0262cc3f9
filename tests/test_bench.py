"""Host logic of bench.py (CPU): the roofline's byte and flop counts against independently
derived figures, the one-GPU rule, and when committed counter traffic is reported.

The expected figures are the I/O floors and flop counts derived by hand from the workload
shapes (inputs and gates read once, the fp32 output and final state written once; flops
B*H*L*(4 Dk Dv + (C+1)(Dk+Dv))), not recomputed with bench.py's own formulas.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gated_linear_rnn_chunkwise_amd import inputs as gin  # noqa: E402

W = gin.WORKLOADS


@pytest.mark.parametrize("name,expect", [
    # 262,144 head-tokens x (3 x 256 B bf16 q, k, v + 512 B fp32 per-channel gate + 512 B fp32
    # output) + 128 x 64 KB final state
    ("gla_bf16_B8H16L2048", 262144 * 1792 + 128 * 65536),
    # 262,144 head-tokens x (768 + 512) B, fixed gate (no bytes per token) + 32 final states
    ("retnet_bf16_B4H8L8192", 262144 * 1280 + 32 * 65536),
    # 524,288 head-tokens x 1792 B + 16 final states
    ("long_gla_bf16_H16L32768_C64", 524288 * 1792 + 16 * 65536),
    # 524,288 head-tokens x (2 x 512 B q, k + 1024 B v + 4 B gate + 4 B input gate + 2048 B
    # output) + 64 final states of 256 x 512 fp32
    ("mlstm_sig_bf16_B8H8L8192", 524288 * 4104 + 64 * 524288),
    # fp32, no gate: 256 tokens x (3 x 256 B + 256 B output) + one 16 KB state
    ("ungated_f32_L256", 256 * 1024 + 16384),
])
def test_io_floor_bytes(name, expect):
    assert bench.io_floor_bytes(W[name]) == expect


@pytest.mark.parametrize("name,chunk,gflop", [
    ("gla_bf16_B8H16L2048", 64, 21.54),
    ("retnet_bf16_B4H8L8192", 128, 25.84),
    ("long_gla_bf16_H16L32768_C64", 64, 43.08),
    ("long_gla_bf16_H16L32768_C256", 256, 68.85),
    ("mlstm_sig_bf16_B8H8L8192", 256, 378.36),
])
def test_algorithmic_flops(name, chunk, gflop):
    assert abs(bench.algorithmic_flops(W[name], chunk) / 1e9 - gflop) < 0.006


def test_more_than_one_gpu_exits_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    rec = {"gla_bf16_B8H16L2048": {"kernel_source_sha256_16": bench.kernel_source_hash("gla"),
                                   "bytes_per_launch": 123},
           "retnet_bf16_B4H8L8192": {"kernel_source_sha256_16": "0000000000000000", "bytes_per_launch": 456}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("gla_bf16_B8H16L2048") == 123
    assert bench.measured_traffic("retnet_bf16_B4H8L8192") is None   # other kernel source
    assert bench.measured_traffic("long_gla_bf16_H16L32768_C64") is None  # not profiled
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("gla_bf16_B8H16L2048") is None
