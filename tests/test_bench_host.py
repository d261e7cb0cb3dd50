"""bench.py's host logic on the CPU (no GPU): the one-GPU contract, skew selection, the
per-expert roofline and the source hashes the traffic records are keyed by."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mixture_experts_routed_router_amd import inputs  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_pick_skew():
    w = inputs.WORKLOADS["qwen3_30b_a3b_shaped"]
    assert bench.pick_skew(w, None) == w.skews[len(w.skews) // 2]
    assert bench.pick_skew(w, "0.8") == 0.8
    assert bench.pick_skew(w, "hot4") == "hot4"
    with pytest.raises(SystemExit):
        bench.pick_skew(w, "0.3")


def test_ffn_roofline_by_hand():
    w = inputs.WORKLOADS["olmoe_shaped"]
    H, I = w.H, w.I
    # one expert with many rows (MFMA-bound), one with 1 row (weight-bound), one untouched
    n = [100000, 1, 0]
    t, touched, wbytes, bound = bench.ffn_roofline(w, n, 2)
    per_flop = 6.0 * H * I / (bench.PEAK_BF16_TFLOPS * 1e12)
    per_expert_bytes = 3.0 * H * I * 2
    expect = 100000 * per_flop + per_expert_bytes / (bench.PEAK_HBM_GBS * 1e9)
    assert abs(t - expect) <= 1e-12 * expect
    assert touched == 2 and wbytes == 2 * per_expert_bytes
    assert bound == "mfma"
    # the MX weights (17/32 byte per value) against the fp8 peak
    t_mx, _, wb_mx, _ = bench.ffn_roofline(w, n, 17.0 / 32.0, bench.PEAK_FP8_TFLOPS)
    assert wb_mx == 2 * 3.0 * H * I * 17.0 / 32.0
    assert t_mx < t


def test_source_hashes_cover_the_kernel_files():
    a, b = bench.ffn_source_sha256("bf16"), bench.ffn_source_sha256("mx")
    assert len(a) == 64 and len(b) == 64 and a != b
