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


def _write_pmc_csv(path, kernel, dispatches):
    """A p_counter_collection.csv as rocprofv3 writes it: one row per
    (dispatch, counter, dimension instance)."""
    import csv
    os.makedirs(path, exist_ok=True)
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        wr.writerow(cols)
        for did, (dur_ns, counters) in enumerate(dispatches, 1):
            for cname, (value, parts) in counters.items():
                for _ in range(parts):  # the value split over dimension instances
                    wr.writerow([did, did, "Agent 1", 1, 1, 1, 131072, 1, kernel, 512, 0, 0, 256, 0, 32,
                                 cname, value / parts, 1000, 1000 + dur_ns])


def test_counter_summary_normalisation(tmp_path):
    """GRBM_GUI_ACTIVE is summed over 8 XCDs and SQ counters over 32 shader
    engines: a 50 us dispatch at 2.0 GHz (1e5 cycles per XCD) whose 1024
    SIMDs keep the matrix cores busy 40% of the time reads back as 2.0 GHz
    and 40% MFMA busy."""
    kern = "_ZN12_GLOBAL__N_115attn_fwd_kernelIDF16b"
    cyc = 1.0e5
    n_mfma = 0.4 * 1024 * cyc / 32
    sq = {"GRBM_GUI_ACTIVE": (8 * cyc, 8), "SQ_CYCLES": (32 * cyc, 32),
          "SQ_VALU_MFMA_BUSY_CYCLES": (32 * n_mfma, 32), "SQ_INSTS_VALU_MFMA_MOPS_BF16": (n_mfma * 64, 32),
          "SQ_INSTS_MFMA": (n_mfma, 32), "SQ_INSTS_VALU": (7.5 * n_mfma, 32), "SQ_INSTS_LDS": (1.5 * n_mfma, 32),
          "SQ_LDS_BANK_CONFLICT": (0.0, 32), "SQ_LDS_IDX_ACTIVE": (1e6, 32)}
    wait = {"GRBM_GUI_ACTIVE": (8 * cyc, 8), "SQ_WAVE_CYCLES": (1e7, 32), "SQ_WAIT_ANY": (3.5e6, 32),
            "SQ_ACTIVE_INST_ANY": (3e6, 32), "SQ_ACTIVE_INST_VALU": (2e6, 32), "SQ_ACTIVE_INST_LDS": (4e5, 32),
            "SQ_ACTIVE_INST_VMEM": (1e5, 32), "SQ_VALU_MFMA_COEXEC_CYCLES": (0.5 * 32 * n_mfma, 32),
            "SQ_INST_CYCLES_VMEM_RD": (1e5, 32), "TA_TA_BUSY": (0.3 * 256 * cyc, 256)}
    name = bench.DEFAULT_WORKLOAD
    _write_pmc_csv(str(tmp_path / f"pmc_sq_{name}"), kern, [(50_000, sq)] * 3)
    _write_pmc_csv(str(tmp_path / f"pmc_wait_{name}"), kern, [(50_000, wait)] * 3)
    bench.write_counters(str(tmp_path), name, out_dir=str(tmp_path))
    import json
    c = json.load(open(tmp_path / f"counters_{name}.json"))
    assert abs(c["shader_clock_ghz"] - 2.0) < 1e-9
    assert abs(c["mfma_busy_pct"] - 40.0) < 1e-9
    assert abs(c["sq_cycles_per_se_over_xcd_cycles"] - 1.0) < 1e-9
    assert abs(c["valu_insts_per_mfma"] - 7.5) < 1e-9
    assert abs(c["wave_waiting_pct"] - 35.0) < 1e-9
    assert abs(c["ta_busy_pct"] - 30.0) < 1e-9
    assert abs(c["mfma_coexec_over_mfma_busy"] - 0.5) < 1e-9
    assert abs(c["mfma_flops_per_dispatch"] - n_mfma * 64 * 512) < 1e-3
    assert (tmp_path / f"attn_fwd_{name}_counters.md").exists()


def test_traffic_summary_scaling(tmp_path):
    """Each counter is scaled by what it reads for the 512 MiB copy."""
    name = "gqa_llama2_70b"
    kern = "_ZN12_GLOBAL__N_115attn_fwd_kernelIDF16b"
    copy = "__amd_rocclr_copyBuffer"
    kib = (1 << 29) / 1024
    _write_pmc_csv(str(tmp_path / f"fetch_{name}"), kern, [(10, {"FETCH_SIZE": (1000.0, 16)})] * 2)
    _write_pmc_csv(str(tmp_path / f"write_{name}"), kern, [(10, {"WRITE_SIZE": (300.0, 16)})] * 2)
    _write_pmc_csv(str(tmp_path / "fetch_copy"), copy, [(10, {"FETCH_SIZE": (kib / 2, 16)})] * 3)
    _write_pmc_csv(str(tmp_path / "write_copy"), copy, [(10, {"WRITE_SIZE": (kib, 16)})] * 3)
    bench.write_traffic(str(tmp_path), name, out_dir=str(tmp_path))
    import json
    t = json.load(open(tmp_path / f"traffic_{name}.json"))
    assert abs(t["fetch_scale"] - 2.0) < 1e-12 and abs(t["write_scale"] - 1.0) < 1e-12
    assert abs(t["traffic_bytes_per_launch"] - (2000.0 + 300.0) * 1024) < 1e-6
