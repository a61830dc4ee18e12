"""bench.py's host-side contract, checked on the CPU: one GPU only (N > 1
exits with a message), a clear exit without a GPU, and the metric's FLOP and
algorithmic-byte counts for the benchmark workload."""

import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_attention_06_amd import workloads as W  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_exits_with_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_gpu_exits_cleanly():
    if torch.cuda.is_available():
        return
    r = _run("--steps", "1", "--warmup", "1")
    assert r.returncode == 1 and "needs a GPU" in r.stderr


def test_metric_counts_for_the_benchmark_workload():
    w = W.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (w.B, w.S, w.Hq, w.Hkv, w.D, w.dtype, w.causal) == (1, 2048, 32, 32, 128, "bf16", True)
    # 4·B·H·S²·D halved for causal = 34.36 GFLOP
    assert bench.metric_flops(w) == 4 * 1 * 32 * 2048 ** 2 * 128 / 2 == 34359738368
    # Q, K, V read once and O written once, bf16: 4 · 2048 · 32 · 128 · 2 B = 64 MiB
    assert bench.min_hbm_bytes(w, None) == 64 * 2 ** 20


def test_padded_workload_algorithmic_counts():
    """Key padding: the metric keeps the dense count; the algorithmic FLOPs
    and bytes count only the L_b visible keys of each batch entry."""
    w = W.WORKLOADS["batched_padded"]
    pad = [128, 512] + [320] * (w.B - 2)
    dense = bench.metric_flops(w)
    assert dense == 4 * w.B * w.Hq * w.S ** 2 * w.D
    assert bench.algorithmic_flops(w, pad) == sum(4 * w.Hq * w.S * L * w.D for L in pad)
    el = 2
    assert bench.min_hbm_bytes(w, pad) == 2 * w.B * w.S * w.Hq * w.D * el + 2 * sum(pad) * w.Hkv * w.D * el
    assert bench.algorithmic_flops(w, None) == dense


def test_host_info_names_the_cpu():
    h = bench.host_info()
    assert h["affinity_cores"] >= 1 and h["blas_threads"] >= 1
    assert isinstance(h["cpu_model"], str) and isinstance(h["blas"], str)
