"""Host-side logic of bench.py (CPU): the one-GPU guard, the algorithmic bytes the
roofline fraction is priced on, and the rule that the measured HBM traffic is reported
only for the kernel sources it was taken on."""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import bench
import synth

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_of_the_benchmark_block():
    cfg = synth.CONFIGS["qwen8b_k16"]
    # W in bf16, the 17 hidden rows and gamma in bf16, and the 16 rows of fp32 draft
    # logits that the softmax proposal reads at T > 0.
    w = 151936 * 4096 * 2
    x = 17 * 4096 * 2 + 4096 * 2
    q = 16 * 151936 * 4
    assert bench.algorithmic_bytes(cfg, 1.0, True) == w + x + q == 1_254_531_072
    # at T = 0, or with a point-mass proposal, q is never read
    assert bench.algorithmic_bytes(cfg, 0.0, True) == w + x
    assert bench.algorithmic_bytes(cfg, 1.0, False) == w + x


def test_algorithmic_bytes_fp8_head():
    cfg = synth.CONFIGS["qwen8b_k16_fp8"]
    # one byte per weight plus one fp32 scale per vocabulary row; activations stay bf16
    expect = 151936 * 4096 + 151936 * 4 + 17 * 4096 * 2 + 4096 * 2 + 16 * 151936 * 4
    assert bench.algorithmic_bytes(cfg, 1.0, True) == expect


def test_lmhead_flops():
    cfg = synth.CONFIGS["qwen8b_k32_b4"]
    assert bench.lmhead_flops(cfg) == 2 * 4 * 33 * 151936 * 4096


def test_traffic_is_dropped_when_kernel_sources_change(monkeypatch):
    t = bench.measured_traffic("qwen8b_k16")
    if t is not None:
        # counters at most a few percent above the algorithmic bytes of a launch
        cfg = synth.CONFIGS["qwen8b_k16"]
        a = bench.algorithmic_bytes(cfg, 1.0, True)
        assert a <= t <= 1.1 * a
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("qwen8b_k16") is None


def test_split_d_workloads_are_labelled():
    """The bench names the split-d kernels for the workloads that take them (bf16, 34..144
    rows) and the fused kernel otherwise."""
    assert bench.wide_path(synth.CONFIGS["qwen8b_k32_b4"])
    assert bench.wide_path(synth.CONFIGS["d5120_k32_b2"])
    assert not bench.wide_path(synth.CONFIGS["qwen8b_k16"])
    assert not bench.wide_path(synth.CONFIGS["qwen8b_k16_fp8"])
    assert not bench.wide_path(synth.CONFIGS["tiny"])
