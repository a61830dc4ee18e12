#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

A step is one attn_fwd call (one kernel launch) over one batch of seeded synthetic input of the
Llama-2-7B-shaped causal prefill (B=1, H=32, S=2048, D=128, bf16) with inputs
already resident in device memory.  Throughput counts 4·B·H·S²·D FLOPs,
halved under causal masking, over the wall time of K timed steps (captured
once as a HIP graph and replayed; --no-graph times eager launches); the
roofline block divides the same FLOP count by the kernel's average duration
over the same back-to-back launches, measured with HIP events on the launch
stream.  roofline.traffic is the measured device-memory traffic per launch
(FETCH_SIZE + WRITE_SIZE counters scaled by a plain copy of known size), read
from profiles/traffic_<workload>.json when that file was taken on the current
kernel source, else null.  The cpu_baseline block times the fp64 CPU oracle on
a bounded sample of heads of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--all] [--sweep] [--rope] [--decode] [--varlen] [--masked]
                    [--general-d] [--write-traffic PROF_DIR]
                    [--copy-calibration]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused attention fwd TFLOP/s (bf16, causal) and % of MI355X MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp32": 157.3}  # MI355X dense MFMA
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "llama2_7b_prefill"


def metric_flops(w):
    f = 4.0 * w.B * w.Hq * w.S * w.S * w.D
    return f / 2.0 if w.causal else f


def algorithmic_flops(w, pad):
    """FLOPs of the scores the method actually computes: with key padding,
    batch b has L_b visible keys per row (4·H·S·L_b·D), halved under causal
    masking like the metric's count.  Equals metric_flops without padding."""
    if pad is None:
        return metric_flops(w)
    f = sum(4.0 * w.Hq * w.S * int(min(max(L, 0), w.S)) * w.D for L in pad)
    return f / 2.0 if w.causal else f


def min_hbm_bytes(w, pad):
    """Q, K, V read once, O (and LSE) written once (the score matrix never
    reaches memory); with key padding, K and V rows past L_b are never read."""
    el = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    qo = 2 * w.B * w.S * w.Hq * w.D * el
    rows = w.B * w.S if pad is None else sum(int(min(max(L, 0), w.S)) for L in pad)
    kv = 2 * rows * w.Hkv * w.D * el
    lse = w.B * w.Hq * w.S * 4 if w.want_lse else 0
    return qo + kv + lse


def time_steps(step, steps, warmup, use_graph=True, warmup_s=0.0):
    """Run ``step`` (which launches on the current stream) for an untimed
    warmup of at least ``warmup`` steps and ``warmup_s`` seconds, then time
    exactly ``steps`` steps: captured once as a HIP graph and replayed (or
    launched eagerly), bracketed by HIP events on the launch stream (device
    time per step) and by synchronize + a host clock (wall time per step).
    Returns (wall ms per step, device ms per step, warmup steps done)."""
    import torch
    t_w = time.perf_counter()
    done = 0
    while done < warmup or (warmup_s > 0 and time.perf_counter() - t_w < warmup_s):
        step()
        done += 1
        if done % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            for _ in range(steps):
                step()
        graph.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(steps):
            step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps, done


def run_gpu(w, steps, warmup, use_graph=True, warmup_s=0.0, rope=False):
    import torch
    from transformer_attention_06_amd import attn as A
    from transformer_attention_06_amd import workloads as W

    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    q, k, v, pad = W.make_inputs(w)
    qd = torch.from_numpy(q).to(dt).cuda()
    kd = torch.from_numpy(k).to(dt).cuda()
    vd = torch.from_numpy(v).to(dt).cuda()
    del q, k, v
    pad_d = None if pad is None else torch.from_numpy(pad).cuda()
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda") if w.want_lse else None
    mask = A.ATTN_MASK_NONE if pad is None else A.ATTN_MASK_KEY_PADDING
    k_rot = torch.empty_like(kd) if rope else None
    def step():
        # launches on the current stream (the capture stream while capturing)
        if rope:  # rotary pass over K, then the attention with Q rotated at load
            A.attn_fwd_rope(qd, kd, vd, mask, pad_d, None, w.causal, w.Hq, w.Hkv, None, None, k_rot, out, lse)
        else:
            A.attn_fwd(qd, kd, vd, mask, pad_d, None, w.causal, w.Hq, w.Hkv, out, lse)

    ms_wall, ms_dev, done = time_steps(step, steps, warmup, use_graph, warmup_s)
    return dict(ms_per_step=ms_wall, kernel_ms_mean=ms_dev, pad=pad, warmup_done=done)


def kernel_source_sha():
    """Hash of the library's sources as they stand in the tree (the same
    digest the build embeds in attn_version())."""
    from transformer_attention_06_amd.build import source_hash
    return source_hash()


def check_library_matches_sources():
    """Refuse to report numbers for a library built from other sources."""
    from transformer_attention_06_amd import attn as A
    built, here = A.library_source_hash(), kernel_source_sha()
    if built != here:
        print(f"bench.py: the loaded library was built from sources {built}, the tree holds {here}: "
              "rebuild (python -m transformer_attention_06_amd.build) before measuring.", file=sys.stderr)
        sys.exit(3)
    return here


def measured_traffic(name):
    """Bytes per launch from a committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def measured_counters(name):
    """The derived counter figures of a committed summary, if it is current."""
    path = os.path.join(ROOT, "profiles", f"counters_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_sha") != kernel_source_sha():
        return None
    keys = ("shader_clock_ghz", "mfma_busy_pct", "valu_insts_per_mfma", "lds_insts_per_mfma",
            "lds_bank_conflict_pct", "wave_waiting_pct", "ta_busy_pct")
    return {k: round(c[k], 4) for k in keys} | {"source": f"profiles/counters_{name}.json"}


def copy_calibration(nbytes=1 << 29, reps=3):
    """A plain device-to-device copy of known size, for scaling the memory
    traffic counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "kernel_source_sha": kernel_source_sha()}), flush=True)


def _counter_rows(prof_dir, sub, kernel):
    """Rows of prof_dir/sub/p_counter_collection.csv (one rocprofv3 --pmc
    run) for dispatches of `kernel`, grouped per dispatch: {id: {"name",
    "dur_ns", counter: value summed over the counter's dimensions}}."""
    import csv
    path = os.path.join(prof_dir, sub, "p_counter_collection.csv")
    out = {}
    for r in csv.DictReader(open(path)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = out.setdefault(int(r["Dispatch_Id"]), {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _pmc_cmd(counters, prof_dir, sub, args):
    return f"rocprofv3 --pmc {counters} --output-format csv -d {prof_dir}/{sub} -o p -- python3 bench.py {args}"


def write_traffic(prof_dir, name=DEFAULT_WORKLOAD, out_dir=None):
    """Write profiles/traffic_<name>.json from four rocprofv3 --pmc runs under
    prof_dir (fetch_<name>, write_<name>: the workload; fetch_copy,
    write_copy: the 512 MiB copy calibration), each holding
    p_counter_collection.csv: the attention kernel's FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads for
    the copy of known size."""
    import statistics

    def values(sub, kernel, counter):
        return [d[counter] for d in _counter_rows(prof_dir, sub, kernel).values() if counter in d]

    nbytes_kib = (1 << 29) / 1024.0
    fetch = values(f"fetch_{name}", "attn_fwd_kernel", "FETCH_SIZE")
    write = values(f"write_{name}", "attn_fwd_kernel", "WRITE_SIZE")
    fscale = nbytes_kib / statistics.median(values("fetch_copy", "copyBuffer", "FETCH_SIZE"))
    wscale = nbytes_kib / statistics.median(values("write_copy", "copyBuffer", "WRITE_SIZE"))
    fk, wk = statistics.mean(fetch), statistics.mean(write)
    run = f"--workload {name} --steps 5 --warmup 2 --no-cpu-baseline"
    out = {"workload": name, "kernel_source_sha": kernel_source_sha(),
           "fetch_size_kib_per_dispatch": fk, "write_size_kib_per_dispatch": wk,
           "fetch_scale": fscale, "write_scale": wscale,
           "traffic_bytes_per_launch": (fk * fscale + wk * wscale) * 1024.0,
           "commands": [_pmc_cmd(c, prof_dir, sub, args) for c, sub, args in (
               ("FETCH_SIZE", f"fetch_{name}", run),
               ("WRITE_SIZE", f"write_{name}", run),
               ("FETCH_SIZE", "fetch_copy", "--copy-calibration"),
               ("WRITE_SIZE", "write_copy", "--copy-calibration"))]}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, f"traffic_{name}.json"), "w") as f:
        json.dump(out, f, indent=1)
    from transformer_attention_06_amd import workloads as W
    w = W.WORKLOADS[name]
    pad = W.make_inputs(w)[3] if w.mask_kind else None
    alg = min_hbm_bytes(w, pad)
    md = [f"# Device-memory traffic per launch — {name}", "",
          f"Workload: {name} (B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} {w.dtype}"
          f"{' causal' if w.causal else ''}{' key-padding' if w.mask_kind else ''}{' LSE' if w.want_lse else ''}).",
          f"Kernel source sha256[:16]: `{out['kernel_source_sha']}`.", "",
          "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each in its own rocprofv3 run, from the "
          "repository root:", ""]
    md += [f"- `{c}`" for c in out["commands"]]
    md += ["", f"Summary written by `python3 bench.py --write-traffic {prof_dir} --workload {name}` "
           f"(`profiles/traffic_{name}.json`).", "",
           f"Calibration with a plain 512 MiB device copy (`bench.py --copy-calibration`): FETCH_SIZE x{fscale:.4f}, "
           f"WRITE_SIZE x{wscale:.4f}.", "",
           "| quantity | value |", "|---|---|",
           f"| FETCH_SIZE (KiB per dispatch, mean) | {fk:.1f} |",
           f"| WRITE_SIZE (KiB per dispatch, mean) | {wk:.1f} |",
           f"| scaled read bytes | {fk * fscale / 1024:.2f} MiB |",
           f"| scaled write bytes | {wk * wscale / 1024:.2f} MiB |",
           f"| traffic per launch | {out['traffic_bytes_per_launch'] / 2**20:.2f} MiB |",
           f"| algorithmic minimum (Q, K, V read once (visible keys), O written once, LSE) | {alg / 2**20:.2f} MiB |",
           f"| ratio | {out['traffic_bytes_per_launch'] / alg:.3f} |"]
    with open(os.path.join(out_dir, f"attn_fwd_{name}_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out), flush=True)


# Two counter passes per workload (rocprofv3 collects at most 8 SQ, 2 TA and
# 2 GRBM counters per run).  SQ counters are summed over the 32 shader
# engines (4 per XCD), GRBM_GUI_ACTIVE over the 8 XCDs: one XCD's busy
# cycles are GRBM_GUI_ACTIVE / 8, and that over the dispatch's duration is
# the shader clock.  SQ_VALU_MFMA_BUSY_CYCLES sums the matrix-core busy
# cycles of all 1024 SIMDs, so MFMA busy = it / (1024 x one XCD's cycles).
# The SQ_WAVE_CYCLES / SQ_WAIT_ANY / SQ_ACTIVE_INST_* family counts wave
# cycles in one common unit; only their ratios are used.
PMC_PASSES = {
    "pmc_sq": "SQ_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_{mops} SQ_INSTS_MFMA SQ_INSTS_VALU "
              "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE",
    "pmc_wait": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
                "SQ_ACTIVE_INST_VMEM SQ_VALU_MFMA_COEXEC_CYCLES SQ_INST_CYCLES_VMEM_RD TA_TA_BUSY GRBM_GUI_ACTIVE",
}
N_XCD, N_SIMD, N_CU = 8, 1024, 256


def write_counters(prof_dir, name=DEFAULT_WORKLOAD, out_dir=None):
    """Write profiles/counters_<name>.json and profiles/attn_fwd_<name>_counters.md
    from the two rocprofv3 --pmc passes under prof_dir (pmc_sq_<name>,
    pmc_wait_<name>, each a run of bench.py on the workload)."""
    import statistics
    from transformer_attention_06_amd import workloads as W
    w = W.WORKLOADS[name]
    mops = {"bf16": "BF16", "fp16": "F16", "fp32": "F32"}[w.dtype]
    a = _counter_rows(prof_dir, f"pmc_sq_{name}", "attn_fwd_kernel")
    b = _counter_rows(prof_dir, f"pmc_wait_{name}", "attn_fwd_kernel")
    m = lambda rows, f: statistics.mean(f(d) for d in rows.values())
    cyc_a = lambda d: d["GRBM_GUI_ACTIVE"] / N_XCD
    cyc_b = lambda d: d["GRBM_GUI_ACTIVE"] / N_XCD
    mfma_flops = m(a, lambda d: d[f"SQ_INSTS_VALU_MFMA_MOPS_{mops}"] * 512.0)
    c = {
        "workload": name, "kernel_source_sha": kernel_source_sha(), "dispatches": [len(a), len(b)],
        "dispatch_us_mean": m(a, lambda d: d["dur_ns"] / 1e3),
        "xcd_cycles_mean": m(a, cyc_a),
        "shader_clock_ghz": m(a, lambda d: cyc_a(d) / d["dur_ns"]),
        "sq_cycles_per_se_over_xcd_cycles": m(a, lambda d: d["SQ_CYCLES"] / 32 / cyc_a(d)),
        "mfma_busy_pct": 100.0 * m(a, lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc_a(d))),
        "mfma_flops_per_dispatch": mfma_flops,
        "mfma_flops_over_metric_flops": mfma_flops / metric_flops(w),
        "valu_insts_per_mfma": m(a, lambda d: d["SQ_INSTS_VALU"] / d["SQ_INSTS_MFMA"]),
        "lds_insts_per_mfma": m(a, lambda d: d["SQ_INSTS_LDS"] / d["SQ_INSTS_MFMA"]),
        "lds_bank_conflict_pct": 100.0 * m(a, lambda d: d["SQ_LDS_BANK_CONFLICT"] / max(d["SQ_LDS_IDX_ACTIVE"], 1.0)),
        "wave_waiting_pct": 100.0 * m(b, lambda d: d["SQ_WAIT_ANY"] / d["SQ_WAVE_CYCLES"]),
        "wave_issuing_pct": 100.0 * m(b, lambda d: d["SQ_ACTIVE_INST_ANY"] / d["SQ_WAVE_CYCLES"]),
        "wave_valu_pct": 100.0 * m(b, lambda d: d["SQ_ACTIVE_INST_VALU"] / d["SQ_WAVE_CYCLES"]),
        "wave_lds_pct": 100.0 * m(b, lambda d: d["SQ_ACTIVE_INST_LDS"] / d["SQ_WAVE_CYCLES"]),
        "wave_vmem_pct": 100.0 * m(b, lambda d: d["SQ_ACTIVE_INST_VMEM"] / d["SQ_WAVE_CYCLES"]),
        "mfma_coexec_over_mfma_busy": m(b, lambda d: d["SQ_VALU_MFMA_COEXEC_CYCLES"] / N_SIMD / cyc_b(d)) /
                                      max(m(a, lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cyc_a(d)), 1e-9),
        "ta_busy_pct": 100.0 * m(b, lambda d: d["TA_TA_BUSY"] / (N_CU * cyc_b(d))),
        "commands": [_pmc_cmd(PMC_PASSES[p].format(mops=mops), prof_dir, f"{p}_{name}",
                              f"--workload {name} --steps 5 --warmup 2 --no-cpu-baseline") for p in PMC_PASSES],
    }
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, f"counters_{name}.json"), "w") as f:
        json.dump(c, f, indent=1)
    rows = [
        ("dispatches (pass 1, pass 2)", f"{c['dispatches'][0]}, {c['dispatches'][1]}"),
        ("dispatch duration under counters (µs, mean)", f"{c['dispatch_us_mean']:.2f}"),
        ("busy cycles of one XCD (GRBM_GUI_ACTIVE / 8)", f"{c['xcd_cycles_mean']:.4g}"),
        ("shader clock (XCD cycles / duration, GHz)", f"{c['shader_clock_ghz']:.3f}"),
        ("SQ_CYCLES / 32 shader engines ÷ XCD cycles (consistency)", f"{c['sq_cycles_per_se_over_xcd_cycles']:.3f}"),
        ("MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs × XCD cycles))", f"{c['mfma_busy_pct']:.1f} %"),
        ("MFMA FLOPs / metric FLOPs", f"{c['mfma_flops_over_metric_flops']:.4f}"),
        ("VALU instructions (incl. MFMA) per MFMA", f"{c['valu_insts_per_mfma']:.2f}"),
        ("LDS instructions per MFMA", f"{c['lds_insts_per_mfma']:.2f}"),
        ("LDS bank conflicts (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)", f"{c['lds_bank_conflict_pct']:.2f} %"),
        ("wave cycles waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)", f"{c['wave_waiting_pct']:.1f} %"),
        ("wave cycles issuing any instruction (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES)", f"{c['wave_issuing_pct']:.1f} %"),
        ("  VALU / LDS / VMEM issue (SQ_ACTIVE_INST_* / SQ_WAVE_CYCLES)",
         f"{c['wave_valu_pct']:.1f} / {c['wave_lds_pct']:.1f} / {c['wave_vmem_pct']:.1f} %"),
        ("MFMA cycles with VALU co-issued (SQ_VALU_MFMA_COEXEC_CYCLES / MFMA busy)",
         f"{c['mfma_coexec_over_mfma_busy']:.2f}"),
        ("TA busy (TA_TA_BUSY / (256 CUs × XCD cycles))", f"{c['ta_busy_pct']:.1f} %"),
    ]
    md = [f"# attn_fwd hardware counters — {name}", "",
          f"Workload: {w.name} (B{w.B} Hq{w.Hq} Hkv{w.Hkv} S{w.S} D{w.D} {w.dtype}"
          f"{' causal' if w.causal else ''}{' key-padding' if w.mask_kind else ''}{' LSE' if w.want_lse else ''}).",
          f"Kernel source sha256[:16]: `{c['kernel_source_sha']}`.", "",
          "Two rocprofv3 counter passes, run from the repository root:", ""]
    md += [f"- `{cmd}`" for cmd in c["commands"]]
    md += ["", f"Summary written by `python3 bench.py --write-counters {prof_dir} --workload {name}`; values are means "
           "over the attention kernel's dispatches.", "",
           "Normalisation: SQ counters are summed over the 32 shader engines (4 per XCD) and GRBM_GUI_ACTIVE over "
           "the 8 XCDs, so one XCD's busy cycles are GRBM_GUI_ACTIVE / 8 (SQ_CYCLES / 32 agrees, row 5); those "
           "cycles over the dispatch's duration are the shader clock. SQ_VALU_MFMA_BUSY_CYCLES sums the matrix-core "
           "busy cycles of all 1024 SIMDs (it equals 32 cycles × MFMA instructions here), hence MFMA busy = "
           "SQ_VALU_MFMA_BUSY_CYCLES / (1024 × XCD cycles). The wave-state counters (SQ_WAVE_CYCLES, SQ_WAIT_ANY, "
           "SQ_ACTIVE_INST_*) share one unit and are used only as ratios.", "",
           "| quantity | value |", "|---|---|"]
    md += [f"| {k} | {v} |" for k, v in rows]
    with open(os.path.join(out_dir, f"attn_fwd_{name}_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(c), flush=True)


def cpu_baseline(w, budget_s=12.0):
    """Time the fp64 oracle on whole (batch, head) units of the workload until
    the time budget is spent; report the metric's unit (TFLOP/s)."""
    import oracle
    from transformer_attention_06_amd import workloads as W
    host = host_info()
    import torch
    q, k, v, pad = W.make_inputs(w)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    rnd = lambda x: torch.from_numpy(x).to(dt).to(torch.float32).numpy()
    q, k, v = rnd(q), rnd(k), rnd(v)
    scale = 1.0 / np.sqrt(w.D)
    done = 0
    t0 = time.perf_counter()
    units = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    for (b, h) in units:
        g = oracle.kv_head_for(h, w.Hq, w.Hkv)
        kl = w.S if pad is None else int(pad[b])
        oracle.attention_head(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], scale, w.causal, kl)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    flops = metric_flops(w) * done / len(units)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": f"{done} of {len(units)} (batch, head) units of {w.name}, fp64 numpy, "
                      f"full SxS score matrix, {el:.2f} s wall",
            "host": host}


def host_info():
    """The CPU the oracle runs on: model name, the cores this process may use
    (sched_getaffinity), and the BLAS library numpy calls with its thread
    count (threadpoolctl)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        affinity = os.cpu_count() or 1
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '?')}"
            threads = int(libs[0].get("num_threads", 1))
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return {"cpu_model": model, "affinity_cores": affinity, "blas": blas, "blas_threads": threads}


DECODE_SHAPES = {
    # Llama-2-70B-shaped decode step: one new token per sequence against a
    # 4096-token KV cache (64 query heads sharing 8 kv heads, D = 128, bf16)
    "llama2_70b_decode_b8": dict(B=8, Sq=1, Sk=4096, Hq=64, Hkv=8, D=128),
    "llama2_70b_decode_b2": dict(B=2, Sq=1, Sk=4096, Hq=64, Hkv=8, D=128),
    # Llama-2-7B-shaped (MHA: one query head per kv head, so one real row
    # per workgroup) decode step, 16 sequences
    "llama2_7b_decode_b16": dict(B=16, Sq=1, Sk=4096, Hq=32, Hkv=32, D=128),
}


def bench_decode(name, steps, warmup, use_graph=True, warmup_s=0.0):
    """Decode attention over a KV cache (split-KV, merged by each row group's
    last split inside the same launch): bound by reading
    the cache, so the figure is algorithmic bytes (K, V caches, Q, O, LSE)
    per call against the HBM peak."""
    import torch
    from transformer_attention_06_amd import attn as A
    sh = DECODE_SHAPES[name]
    B, Sq, Sk, Hq, Hkv, D = (sh[x] for x in ("B", "Sq", "Sk", "Hq", "Hkv", "D"))
    g = torch.Generator(device="cuda").manual_seed(7)
    q = torch.randn(B, Sq, Hq, D, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, Sk, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, Sk, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, Sq, device="cuda", dtype=torch.float32)
    ws = torch.zeros(A.decode_workspace_bytes(B, Sq, Hq, D, Sk), dtype=torch.uint8, device="cuda")

    def step():
        A.attn_fwd_decode(q, k, v, None, None, True, Hq, Hkv, out, lse, ws)

    ms_wall, ms_dev, done = time_steps(step, steps, warmup, use_graph, warmup_s)
    nbytes = 2 * B * Sk * Hkv * D * 2 + 2 * B * Sq * Hq * D * 2 + B * Hq * Sq * 4
    gbs = nbytes / (ms_wall * 1e-3) / 1e9
    achieved = nbytes / (ms_dev * 1e-3) / 1e9
    return {"metric": "decode attention over a KV cache: algorithmic HBM GB/s", "value": round(gbs, 2),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": done, "ms_per_step": round(ms_wall, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) query, K cache and V cache)",
            "config": {"workload": name, **sh, "causal": True, "timing": "hip_graph_replay" if use_graph
                       else "eager_launches", "launches_per_call": 1},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "call_us_mean": round(ms_dev * 1e3, 3), "algorithmic_bytes_per_call": nbytes,
                         "workspace_bytes": int(ws.numel())}}


def bench_varlen(steps, warmup, use_graph=True, warmup_s=0.0, name="batched_varlen"):
    """Packed variable-length sequences (attn_fwd_varlen): the batched short
    sequences (16 lengths in [128, 512], 32 heads, D = 64, fp16, non-causal)
    packed with no padding.  The FLOP count is the algorithmic one, Σ_b
    4·H·L_b²·D (no padded row or key exists); the same lengths run through
    attn_fwd's key-padding path (B × 512 rows, padded query rows computed)
    in the same process give the cost of padding."""
    import torch
    from transformer_attention_06_amd import attn as A
    from transformer_attention_06_amd import workloads as W
    w = W.WORKLOADS[name]
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
    q, k, v, cu = W.make_varlen_inputs(w)
    lens = np.diff(cu)
    qd, kd, vd = (torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))
    cu_d = torch.from_numpy(cu.astype(np.int32)).cuda()
    out = torch.empty_like(qd)
    max_len = int(lens.max())

    def step():
        A.attn_fwd_varlen(qd, kd, vd, cu_d, max_len, None, w.causal, w.Hq, w.Hkv, out, None)

    ms_wall, ms_dev, done = time_steps(step, steps, warmup, use_graph, warmup_s)
    # the same sequences padded to S = 512 under key padding
    pq, pk, pv = (torch.zeros((w.B, w.S) + x.shape[1:], dtype=dt, device="cuda") for x in (q, k, v))
    for b in range(w.B):
        pq[b, :lens[b]], pk[b, :lens[b]], pv[b, :lens[b]] = qd[cu[b]:cu[b + 1]], kd[cu[b]:cu[b + 1]], vd[cu[b]:cu[b + 1]]
    pad_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    pout = torch.empty_like(pq)

    def step_pad():
        A.attn_fwd(pq, pk, pv, A.ATTN_MASK_KEY_PADDING, pad_d, None, w.causal, w.Hq, w.Hkv, pout, None)

    _, ms_pad, _ = time_steps(step_pad, steps, warmup, use_graph, warmup_s)
    fl = float(sum(4.0 * w.Hq * float(L) ** 2 * w.D for L in lens))
    if w.causal:
        fl /= 2.0
    el = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
    nbytes = int(cu[-1]) * (2 * w.Hq + 2 * w.Hkv) * w.D * el
    peak = PEAK_TFLOPS[w.dtype]
    achieved = fl / (ms_dev * 1e-3) / 1e12
    return {"metric": "packed variable-length attention: algorithmic TFLOP/s", "value": round(fl / (ms_wall * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": done, "ms_per_step": round(ms_wall, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (seeded lengths in [128, 512], N(0,1) Q, K, V)",
            "config": {"workload": name, "B": w.B, "T": int(cu[-1]), "max_seqlen": max_len, "Hq": w.Hq,
                       "Hkv": w.Hkv, "D": w.D, "causal": w.causal,
                       "timing": "hip_graph_replay" if use_graph else "eager_launches"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(achieved / peak, 4), "traffic": None,
                         "kernel_us_mean": round(ms_dev * 1e3, 3), "flops_per_launch": fl,
                         "min_hbm_bytes_per_launch": nbytes,
                         "hbm_frac": round(nbytes / (ms_dev * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "padded": {"kernel_us_mean": round(ms_pad * 1e3, 3),
                       "algorithmic_tflops": round(fl / (ms_pad * 1e-3) / 1e12, 3),
                       "note": "same sequences through attn_fwd key padding at S = 512"}}


def bench_masked(steps, warmup, use_graph=True, warmup_s=0.0, name=DEFAULT_WORKLOAD):
    """attn_fwd_masked on the Llama-2-7B-shaped causal prefill: a (1, 1, S, S)
    additive mask (N(0,1)·0.5 shifts, -inf above the diagonal) with the causal
    flag on, so the metric's FLOP count (halved for causal) applies; plain
    attn_fwd on the same Q, K, V is timed alongside."""
    import torch
    from transformer_attention_06_amd import attn as A
    from transformer_attention_06_amd import workloads as W
    w = W.WORKLOADS[name]
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[w.dtype]
    q, k, v, _ = W.make_inputs(w)
    qd, kd, vd = (torch.from_numpy(x).to(dt).cuda() for x in (q, k, v))
    rng = np.random.default_rng(w.seed + 100)
    m = (rng.standard_normal((1, 1, w.S, w.S)) * 0.5).astype(np.float32)
    m[0, 0][np.triu(np.ones((w.S, w.S), bool), 1)] = -np.inf
    md = torch.from_numpy(m).to(dt).cuda()
    out = torch.empty_like(qd)

    def step():
        A.attn_fwd_masked(qd, kd, vd, md, None, True, w.Hq, w.Hkv, out, None)

    ms_wall, ms_dev, done = time_steps(step, steps, warmup, use_graph, warmup_s)

    def step_plain():
        A.attn_fwd(qd, kd, vd, A.ATTN_MASK_NONE, None, None, True, w.Hq, w.Hkv, out, None)

    _, ms_plain, _ = time_steps(step_plain, steps, warmup, use_graph, warmup_s)
    fl = metric_flops(w)
    peak = PEAK_TFLOPS[w.dtype]
    el = 2
    # Q, K, V, O once, plus the mask blocks on or below the diagonal
    nbytes = min_hbm_bytes(w, None) + (w.S * (w.S + 1) // 2) * el
    achieved = fl / (ms_dev * 1e-3) / 1e12
    return {"metric": "fused attention fwd with an additive mask tensor: TFLOP/s", "value": round(fl / (ms_wall * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": done, "ms_per_step": round(ms_wall, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (seeded N(0,1) Q, K, V; N(0,1)*0.5 mask with -inf above the diagonal)",
            "config": {"workload": name + "_masked", "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                       "causal": True, "mask_shape": [1, 1, w.S, w.S],
                       "timing": "hip_graph_replay" if use_graph else "eager_launches"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(achieved / peak, 4), "traffic": None,
                         "kernel_us_mean": round(ms_dev * 1e3, 3), "flops_per_launch": fl,
                         "min_hbm_bytes_per_launch": nbytes},
            "attn_fwd_same_inputs": {"kernel_us_mean": round(ms_plain * 1e3, 3),
                                     "tflops": round(fl / (ms_plain * 1e-3) / 1e12, 3)}}


def bench_one(name, steps, warmup, with_cpu, use_graph=True, warmup_s=0.0, rope=False):
    from transformer_attention_06_amd import workloads as W
    w = W.WORKLOADS[name]
    r = run_gpu(w, steps, warmup, use_graph, warmup_s, rope=rope)
    fl = metric_flops(w)
    value = fl / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = fl / (r["kernel_ms_mean"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": r["warmup_done"],
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape; no weights)",
        "config": {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "causal": w.causal, "mask": "key_padding" if w.mask_kind else "none",
                   "lse": w.want_lse, "rope": rope,
                   "timing": "hip_graph_replay" if use_graph else "eager_launches",
                   "pct_of_peak_wall": round(100 * value / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name),
                     "counters": measured_counters(w.name),
                     "kernel_us_mean": round(r["kernel_ms_mean"] * 1e3, 3),
                     "flops_per_launch": fl,
                     "min_hbm_bytes_per_launch": min_hbm_bytes(w, r["pad"]),
                     # the same launch against the HBM roofline (algorithmic bytes
                     # over the kernel time), for shapes near the ridge
                     "hbm_frac": round(min_hbm_bytes(w, r["pad"]) / (r["kernel_ms_mean"] * 1e-3) / 1e9
                                       / HBM_PEAK_GBS, 4)},
        "source_sha": kernel_source_sha(),
    }
    if r["pad"] is not None:
        # key padding: the metric counts every key (dense S x S, as the
        # metric's definition states); the method computes only the visible
        # ones (sum over b of 4 H S L_b D)
        afl = algorithmic_flops(w, r["pad"])
        line["roofline"]["algorithmic_flops_per_launch"] = afl
        line["roofline"]["algorithmic_tflops"] = round(afl / (r["kernel_ms_mean"] * 1e-3) / 1e12, 3)
        line["roofline"]["algorithmic_frac"] = round(afl / (r["kernel_ms_mean"] * 1e-3) / 1e12 / peak, 4)
    if rope:
        # the call is two launches: the K rotation pass (bandwidth-bound: K
        # read and written once) and the attention with Q rotated at load;
        # the plain attention on the same inputs gives the cost of both
        r0 = run_gpu(w, steps, warmup, use_graph, warmup_s, rope=False)
        el = {"bf16": 2, "fp16": 2, "fp32": 4}[w.dtype]
        kbytes = 2 * w.B * w.S * w.Hkv * w.D * el
        extra_us = (r["kernel_ms_mean"] - r0["kernel_ms_mean"]) * 1e3
        line["roofline"]["traffic"] = None
        line["rope"] = {"call_us_mean": round(r["kernel_ms_mean"] * 1e3, 3),
                        "attn_fwd_us_mean": round(r0["kernel_ms_mean"] * 1e3, 3),
                        "extra_us": round(extra_us, 3),
                        "k_pass_bytes": kbytes,
                        "k_pass_min_us_at_8TBps": round(kbytes / (HBM_PEAK_GBS * 1e3), 3)}
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(w)
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 20 steps and 0.5 s)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="one line per workload (no CPU leg)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of a replayed HIP graph of the K steps")
    ap.add_argument("--write-traffic", metavar="PROF_DIR",
                    help="write profiles/traffic_<workload>.json from the four rocprofv3 --pmc runs under PROF_DIR "
                         "(no GPU needed)")
    ap.add_argument("--write-counters", metavar="PROF_DIR",
                    help="write profiles/counters_<workload>.json and its .md summary from the two rocprofv3 --pmc "
                         "passes under PROF_DIR (no GPU needed)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 512 MiB device copy (counter calibration) and exit")
    ap.add_argument("--decode", action="store_true",
                    help="decode attention over a KV cache (attn_fwd_decode), Llama-2-70B shapes, HBM roofline")
    ap.add_argument("--general-d", action="store_true",
                    help="head dims other than 64 and 128 (D = 80, 96, 112, 144, 160, 192, 256) at B=1, H=32, S=2048, "
                         "bf16, causal; D = 128 (the tuned kernel) for reference")
    ap.add_argument("--masked", action="store_true",
                    help="additive mask tensor (attn_fwd_masked) on the Llama-2-7B-shaped prefill")
    ap.add_argument("--varlen", action="store_true",
                    help="packed variable-length sequences (attn_fwd_varlen) vs the same lengths padded")
    ap.add_argument("--rope", action="store_true",
                    help="time attn_fwd_rope (rotary embedding of Q and K fused with the attention)")
    ap.add_argument("--sweep", action="store_true",
                    help="sequence-length sweep S = 1K..16K at B=1, H=32, D=128, bf16, causal "
                         "(one line per S; an MFMA-bound kernel's time grows as S^2)")
    args = ap.parse_args()
    warmup_s = 0.5 if args.warmup is None else 0.0
    if args.warmup is None:
        args.warmup = 20
    if args.write_traffic:
        write_traffic(args.write_traffic, args.workload)
        return
    if args.write_counters:
        write_counters(args.write_counters, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X).", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    check_library_matches_sources()
    if args.decode:
        for name in DECODE_SHAPES:
            print(json.dumps(bench_decode(name, args.steps, args.warmup, not args.no_graph, warmup_s)), flush=True)
        return
    if args.general_d:
        from transformer_attention_06_amd import workloads as W
        for D in (80, 96, 112, 128, 144, 160, 192, 256):
            w = W.Workload(f"llama2_7b_prefill_d{D}", 1, B=1, S=2048, Hq=32, Hkv=32, D=D, dtype="bf16", causal=True)
            W.WORKLOADS[w.name] = w
            line = bench_one(w.name, args.steps, args.warmup, False, not args.no_graph, warmup_s)
            line["config"]["kernel"] = ("tuned" if D in (64, 128) else "tuned, LDS rows of 128 dims" if D < 128
                                        else "tuned, 32-key tiles, LDS rows of 256 dims" if D <= 160
                                        else "tuned, 32-key tiles, one wavefront per SIMD, AGPR accumulators")
            print(json.dumps(line), flush=True)
        return
    if args.masked:
        print(json.dumps(bench_masked(args.steps, args.warmup, not args.no_graph, warmup_s)), flush=True)
        return
    if args.varlen:
        print(json.dumps(bench_varlen(args.steps, args.warmup, not args.no_graph, warmup_s)), flush=True)
        return
    if args.sweep:
        from transformer_attention_06_amd import workloads as W
        base = None
        for S in (1024, 2048, 4096, 8192, 16384):
            w = W.Workload(f"s_sweep_{S}", 4, B=1, S=S, Hq=32, Hkv=32, D=128, dtype="bf16", causal=True)
            W.WORKLOADS[w.name] = w
            line = bench_one(w.name, max(10, args.steps // (S // 1024)), args.warmup, False, not args.no_graph,
                             warmup_s)
            us = line["roofline"]["kernel_us_mean"]
            base = base or (S, us)
            line["config"]["time_vs_S2_scaling"] = round(us / (base[1] * (S / base[0]) ** 2), 3)
            print(json.dumps(line), flush=True)
        return
    if args.all:
        from transformer_attention_06_amd import workloads as W
        for name in W.WORKLOADS:
            if name == "batched_varlen":  # packed inputs: --varlen
                continue
            print(json.dumps(bench_one(name, args.steps, args.warmup, False, not args.no_graph, warmup_s)), flush=True)
        print(json.dumps(bench_one(DEFAULT_WORKLOAD, args.steps, args.warmup, False, not args.no_graph, warmup_s,
                                   rope=True)), flush=True)
        return
    print(json.dumps(bench_one(args.workload, args.steps, args.warmup, not args.no_cpu_baseline and not args.rope,
                               not args.no_graph, warmup_s, rope=args.rope)), flush=True)


if __name__ == "__main__":
    main()
